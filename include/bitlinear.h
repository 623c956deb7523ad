/*
 * bitlinear.h -- C ABI of libbitlinear.so: the BitNet b1.58 BitLinear forward on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (abbreviations used below):
 *   [HF-1.58]    "Fine-tuning LLMs to 1.58 bits: extreme quantization with BitNet"
 *                (summary of the Hugging Face post, agentlenshq.com)
 *   [bitnet.cpp] "Microsoft's inference framework brings 1-bit large language models
 *                to local devices" (unite.ai)
 *   [b1.58]      "[Paper review] The Era of 1-bit LLMs: All Large Language Models are
 *                in 1.58 Bits" (nubint.ai)
 *
 * The forward is split the way the pages split it: an offline weight conversion into
 * packed 2-bit codes ([HF-1.58] "Key findings"; [bitnet.cpp] the i2_s conversion of
 * "Build and prepare the project"), then per call "quantize the input, run the
 * low-bit matrix product, multiply by the scale" ([bitnet.cpp] "CPU optimization",
 * bitlinear_forward). Activation quantization is its own call so that projections
 * that read the same input (q/k/v, gate/up) quantize it once.
 *
 * Conventions shared by every entry point:
 *   - Shapes follow nn.Linear: W is [N out, K in] row-major (K contiguous), X is
 *     [T tokens, K] row-major, Y = X W^T is [T, N] row-major.
 *   - Every array pointer is a DEVICE pointer owned by the caller; the library keeps
 *     no pointer after the stream-ordered work that uses it has finished, keeps no
 *     device state, and allocates no device memory. The one exception is the static
 *     scratch array of bitlinear_forward_grouped_noalloc (64 MiB per GPU, present
 *     while the library is loaded; no call allocates or frees it).
 *   - Every compute call is asynchronous on `stream` (NULL = the default stream) and
 *     performs no host synchronization; scales stay on the device.
 *   - Arguments are validated on the host before anything is launched; an invalid call
 *     returns its status without touching the GPU, so validation is testable without
 *     one. BL_ERR_HIP reports a failed launch (text from bitlinear_last_hip_error()).
 *   - Data-dependent conditions are not reported: with NaN or Inf inputs the values
 *     written are unspecified, but every kernel still terminates.
 *   - Array base pointers must be 16-byte aligned (BL_ERR_ALIGN otherwise).
 *   - Calls on distinct streams with distinct output buffers may run concurrently.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bl_stream_t; /* the same handle type as hipStream_t */

typedef enum bl_status {
  BL_OK = 0,
  BL_ERR_NULL = 1,         /* a required pointer is NULL */
  BL_ERR_DIM = 2,          /* T, N or K <= 0, or K not a multiple of 4 */
  BL_ERR_K_TOO_LARGE = 3,  /* K > BL_MAX_K */
  BL_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than its query returned */
  BL_ERR_ALIGN = 5,        /* an array base pointer is not 16-byte aligned */
  BL_ERR_HIP = 6,          /* a HIP call failed */
  BL_ERR_ARG = 7           /* another invalid argument (flags, eps, count, kernel) */
} bl_status;

/* Largest K: |acc| <= 127*K must stay below 2^24 so that the int32 accumulator
 * converts to fp32 exactly in the rescale (127 * 132104 = 16,777,208 < 2^24). */
#define BL_MAX_K 132104
/* Largest number of entries in one grouped call. */
#define BL_MAX_GROUP 8
/* bitlinear_quantize_acts flag: skip RMSNorm and quantize X itself (y = x). */
#define BL_NO_NORM 0x1u
#define BL_ABI_VERSION 1

/* Kernel selection for bitlinear_forward_ex (BL_KERNEL_AUTO is what
 * bitlinear_forward uses). */
typedef enum bl_kernel {
  BL_KERNEL_AUTO = 0,
  BL_KERNEL_GEMV = 1,     /* decode GEMV, int8 dot4; needs T == 1 and K % 64 == 0 */
  BL_KERNEL_SKINNY = 2,   /* skinny int8 MFMA GEMM; needs T <= 128, K % 256 == 0 and
                             N < 2^23 (passes of 64 tokens) */
  BL_KERNEL_PREFILL = 3,  /* LDS-tiled int8 MFMA GEMM; needs K % 128 == 0 */
  BL_KERNEL_GENERIC = 4   /* any K % 4 == 0, any T: one thread per output */
} bl_kernel;

/* ---------------------------------------------------------------- weights
 *
 * Absmean ternary quantization and 2-bit packing ([HF-1.58] "How quantization
 * works", weights: per-tensor scale = reciprocal of the mean absolute value, then
 * scale, round, clamp to [-1, 1]; [b1.58] "Proposed method", absmean; packing four
 * codes per int8, [HF-1.58] "Key findings"). Computes, exactly as specified:
 *   S      = sum of |W| over all N*K entries, exact, rounded once to fp64
 *   gamma  = S / (N*K) in fp64;  beta = fp32(gamma) (round to nearest even)
 *   q      = clamp(rint(w * fp32(1/beta)), -1, 1), w * (1/beta) one fp32 product,
 *            rint rounding half to even; all codes 0 when beta < FLT_MIN
 *   packed = byte j of row o holds code k = 4j+i in bits [2i+1:2i] as u = q+1 (0..2)
 * Arguments:
 *   W          device fp32 [N, K], 16-byte aligned; read only
 *   W_packed   device uint8 [N, K/4]; written
 *   w_scale    device fp32 [1]; receives beta
 *   w_gamma    device fp64 [1] or NULL; receives gamma
 *   workspace  device scratch of at least bitlinear_weight_workspace_bytes(N, K)
 *              bytes, 16-byte aligned; contents on entry are ignored
 * The result is independent of launch order and bit-for-bit reproducible. */
size_t bitlinear_weight_workspace_bytes(int64_t N, int64_t K);
bl_status bitlinear_quantize_weights(const float* W, int64_t N, int64_t K,
                                     uint8_t* W_packed, float* w_scale, double* w_gamma,
                                     void* workspace, size_t workspace_bytes,
                                     bl_stream_t stream);

/* ---------------------------------------------------------------- activations
 *
 * Fused RMSNorm + per-token absmax int8 quantization ([b1.58] "Proposed method",
 * RMSNorm; [HF-1.58] "How quantization works", activations: a norm before the
 * quantizer, absmax per token into [-128, 127]; [bitnet.cpp] "2. Activation
 * quantization", gamma = ||x||_inf and an epsilon). Per token t:
 *   ss  = sum_k x_k^2 in fp64 (each square exact; accumulated in double-double
 *         and returned as the rounded sum of its two parts: the correctly rounded
 *         sum except when the exact sum lies within about 2^-100 (relative) of a
 *         rounding midpoint)
 *   r   = 1 / sqrt(ss / K + eps) in fp64 (IEEE division and square root)
 *   y_k = fp32((x_k * r) * g_k), both products in fp64 (no g product when gain is NULL)
 *   s_t = 127 / max(max_k |y_k|, 1e-5) in fp32
 *   Xq  = clamp(rint(y_k * s_t), -128, 127), y_k * s_t one fp32 product
 * With BL_NO_NORM in flags, y = x (gain and eps are ignored).
 * Arguments:
 *   X        device fp32 [T, K], 16-byte aligned
 *   gain     device fp32 [K], 16-byte aligned, or NULL (unit gain)
 *   eps      finite, >= 0 (1e-6 in the Llama-shaped workloads)
 *   Xq       device int8 [T, K]; written
 *   x_scale  device fp32 [T]; receives s_t */
bl_status bitlinear_quantize_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                  float eps, uint32_t flags, int8_t* Xq, float* x_scale,
                                  bl_stream_t stream);

/* One entry of a grouped activation quantization: all entries share T, eps, flags. */
typedef struct bl_act_desc {
  const float* X;     /* device fp32 [T, K] */
  const float* gain;  /* device fp32 [K], 16-byte aligned, or NULL */
  int8_t* Xq;         /* device int8 [T, K] */
  float* x_scale;     /* device fp32 [T] */
  int64_t K;
} bl_act_desc;

/* bitlinear_quantize_acts over `count` (1..BL_MAX_GROUP) independent inputs in one
 * launch; each entry computes exactly what bitlinear_quantize_acts computes. */
bl_status bitlinear_quantize_acts_grouped(const bl_act_desc* descs, int count, int64_t T,
                                          float eps, uint32_t flags, bl_stream_t stream);

/* ---------------------------------------------------------------- forward
 *
 * Ternary x int8 product with exact integer accumulation and the rescale
 * ([HF-1.58] "Computation paradigm": integer additions in place of multiply-adds;
 * "Inference optimization and custom kernels": weights unpacked on the fly inside
 * the product; [bitnet.cpp] "3. BitLinear operation": multiply by the weight scale
 * and the activation dequantization factor; no bias, [b1.58] "Proposed method"):
 *   acc[t, o] = sum_k Xq[t, k] * q[o, k]        (exact, int32)
 *   Y[t, o]   = fp32(acc) * fp32(beta / s_t)    (fp32; within 2 roundings of the
 *                                                exact acc * beta / s_t)
 * Arguments:
 *   Xq, x_scale  outputs of bitlinear_quantize_acts: int8 [T, K], fp32 [T]
 *   W_packed     uint8 [N, K/4] from bitlinear_quantize_weights; w_scale fp32 [1]
 *   Y            device fp32 [T, N]; written
 *   acc          device int32 [T, N] or NULL; receives the exact accumulators
 * K <= BL_MAX_K. Byte patterns 0b11 in W_packed are outside the format; their
 * contribution is unspecified. */
bl_status bitlinear_forward(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                            const uint8_t* W_packed, const float* w_scale, int64_t N,
                            float* Y, int32_t* acc, bl_stream_t stream);

/* bitlinear_forward with an explicit kernel choice (for tests and measurement).
 * Returns BL_ERR_ARG when the chosen kernel does not support the shape. */
bl_status bitlinear_forward_ex(const int8_t* Xq, const float* x_scale, int64_t T,
                               int64_t K, const uint8_t* W_packed, const float* w_scale,
                               int64_t N, float* Y, int32_t* acc, bl_kernel kernel,
                               bl_stream_t stream);

/* The kernel bitlinear_forward would run for this shape. */
bl_kernel bitlinear_forward_choice(int64_t T, int64_t N, int64_t K);

/* Split-K workspace. With up to 128 tokens and few row tiles (for example T = 32..64
 * on a 70B down projection, N = 8192, K = 28672) the tiled MFMA GEMM cuts K into slices
 * so that every CU gets work; each slice writes its exact int32 partial products to a
 * workspace, and a second kernel sums them and applies the rescale (the results are
 * those of bitlinear_forward, bit for bit for acc). The library allocates nothing for
 * this: the caller passes the workspace.
 *
 * bitlinear_forward_workspace_bytes: bytes of workspace that let bitlinear_forward_ws
 * split K for this shape (0: the shape never splits, or invalid dimensions).
 *
 * bitlinear_forward_ws: bitlinear_forward_ex with a workspace (device memory, 16-byte
 * aligned, owned by the caller, not read before it is written, contents undefined after
 * the call; NULL or fewer than bitlinear_forward_workspace_bytes bytes: no split). Calls
 * that share one workspace must not overlap (use it on one stream, or give each stream
 * its own). BL_ERR_ALIGN for a misaligned workspace.
 *
 * bitlinear_forward_grouped_ws: bitlinear_forward_grouped with a workspace; the
 * projections that split run one after another, so the largest of their
 * bitlinear_forward_workspace_bytes is enough.
 *
 * bitlinear_forward_choice_ws: the kernel bitlinear_forward_ws would run with a
 * workspace of that many bytes. */
size_t bitlinear_forward_workspace_bytes(int64_t T, int64_t N, int64_t K);
bl_status bitlinear_forward_ws(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                               const uint8_t* W_packed, const float* w_scale, int64_t N,
                               float* Y, int32_t* acc, bl_kernel kernel, void* workspace,
                               size_t workspace_bytes, bl_stream_t stream);
bl_kernel bitlinear_forward_choice_ws(int64_t T, int64_t N, int64_t K, size_t workspace_bytes);

/* One projection of a grouped forward: all entries share T. */
typedef struct bl_proj_desc {
  const int8_t* Xq;         /* int8 [T, K] */
  const float* x_scale;     /* fp32 [T] */
  const uint8_t* W_packed;  /* uint8 [N, K/4] */
  const float* w_scale;     /* fp32 [1] */
  float* Y;                 /* fp32 [T, N] */
  int32_t* acc;             /* int32 [T, N] or NULL */
  int64_t N;
  int64_t K;
} bl_proj_desc;

/* bitlinear_forward over `count` (1..BL_MAX_GROUP) projections, each with its own
 * weights, scale, input and output (for example q/k/v, or the seven projections of a
 * decoder layer), in as few launches as the shapes allow (one per distinct K on the
 * decode path). Each entry's results are those of bitlinear_forward. */
bl_status bitlinear_forward_grouped(const bl_proj_desc* descs, int count, int64_t T,
                                    bl_stream_t stream);
bl_status bitlinear_forward_grouped_ws(const bl_proj_desc* descs, int count, int64_t T,
                                       void* workspace, size_t workspace_bytes,
                                       bl_stream_t stream);

/* bitlinear_forward_grouped_noalloc: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The same results and kernels as bitlinear_forward_grouped_ws, with the
 * split-K workspace taken from a library-owned device array of
 * BL_NOALLOC_SCRATCH_BYTES (64 MiB) instead of an argument. The array is static: each
 * GPU the library runs on holds its own copy until the process ends, and nothing is
 * allocated or freed by the call. The caller still owns every input and output.
 *   - The first call on a device (with that device current) looks up the array's
 *     address there once; make that first call outside a stream capture.
 *   - Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 *     (two streams, or two threads) race on it and give undefined results. The array
 *     needs no clearing: each split writes its partial products before they are read.
 *   - BL_ERR_WORKSPACE, before any launch, when a projection's split would need more
 *     than BL_NOALLOC_SCRATCH_BYTES (bitlinear_forward_workspace_bytes); BL_ERR_HIP
 *     when the address lookup fails (the message names the call). */
#define BL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bl_status bitlinear_forward_grouped_noalloc(const bl_proj_desc* descs, int count, int64_t T,
                                            bl_stream_t stream);

/* ---------------------------------------------------------------- weight scale groups
 *
 * Group quantization ([bitnet.cpp] "Group quantization and normalization": weights and
 * activations are split into G groups whose parameters are estimated separately, so
 * that no group needs another's). The weights are cut into G blocks of N/G consecutive
 * output rows (a tensor-parallel shard each); every block is quantized exactly as
 * bitlinear_quantize_weights quantizes a whole matrix, with its own beta_g. Activation
 * scales are per token already (bitlinear_quantize_acts). The forward is that of
 * bitlinear_forward with row o rescaled by the scale of its block:
 *   Y[t, o] = fp32(acc) * fp32(beta_{o / (N/G)} / s_t)
 * Arguments as for bitlinear_quantize_weights / bitlinear_forward_ex, plus:
 *   G        1 <= G, N % G == 0 (G = 1 is the per-tensor quantizer); else BL_ERR_ARG
 *   w_scale  device fp32 [G] (beta per block); w_gamma fp64 [G] or NULL
 * The quantizer runs the per-tensor kernels once per block on the stream. */
bl_status bitlinear_quantize_weights_scale_groups(const float* W, int64_t N, int64_t K, int64_t G,
                                                  uint8_t* W_packed, float* w_scale,
                                                  double* w_gamma, void* workspace,
                                                  size_t workspace_bytes, bl_stream_t stream);
bl_status bitlinear_forward_scale_groups(const int8_t* Xq, const float* x_scale, int64_t T,
                                         int64_t K, const uint8_t* W_packed, const float* w_scale,
                                         int64_t N, int64_t G, float* Y, int32_t* acc,
                                         bl_kernel kernel, bl_stream_t stream);
/* bitlinear_forward_grouped where entry i has groups[i] weight scale groups. */
bl_status bitlinear_forward_grouped_scale_groups(const bl_proj_desc* descs, const int64_t* groups,
                                                 int count, int64_t T, bl_stream_t stream);

/* ---------------------------------------------------------------- 1-bit sign variant
 *
 * The original BitNet weight binarization ([bitnet.cpp] "1. Weight binarization":
 * W_f = Sign(W - alpha) with alpha the mean of W and Sign(x) = +1 for x > 0, -1
 * otherwise; [BitDelta] Eq. (2) is the same rule and Eq. (4) gives mean |W| as the
 * scale of a sign code). Activations are quantized by bitlinear_quantize_acts; the
 * rescale is that of bitlinear_forward. Computes:
 *   alpha = (exact sum of W, rounded once to fp64) / (N*K) in fp64
 *   c     = +1 where fp64(w) > alpha, else -1 (an exact comparison)
 *   beta  = fp32(mean |W|), as in bitlinear_quantize_weights
 *   bits  = bit i of byte j of row o holds code k = 8j+i, 1 for +1 and 0 for -1
 * Arguments:
 *   W          device fp32 [N, K], K % 8 == 0, 16-byte aligned; read only
 *   W_bits     device uint8 [N, K/8], 16-byte aligned; written
 *   w_scale    device fp32 [1]; receives beta
 *   w_alpha    device fp64 [1] or NULL; receives alpha
 *   workspace  as for bitlinear_quantize_weights (the same size covers both) */
bl_status bitlinear_quantize_weights_sign(const float* W, int64_t N, int64_t K,
                                          uint8_t* W_bits, float* w_scale, double* w_alpha,
                                          void* workspace, size_t workspace_bytes,
                                          bl_stream_t stream);

/* acc[t, o] = sum_k Xq[t, k] * c[o, k] (exact, int32), Y = fp32(acc) * fp32(beta / s_t).
 * W_bits uint8 [N, K/8] from bitlinear_quantize_weights_sign, K % 8 == 0. T == 1 with
 * K % 128 == 0 runs the decode GEMV, any other shape a one-thread-per-output kernel. */
bl_status bitlinear_forward_sign(const int8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                                 const uint8_t* W_bits, const float* w_scale, int64_t N,
                                 float* Y, int32_t* acc, bl_stream_t stream);

/* bitlinear_forward_sign over `count` (1..BL_MAX_GROUP) projections (W_packed of each
 * entry holds sign bits, [N, K/8]); one launch per kernel kind. */
bl_status bitlinear_forward_sign_grouped(const bl_proj_desc* descs, int count, int64_t T,
                                         bl_stream_t stream);

/* ---------------------------------------------------------------- training side
 *
 * Fake quantization with the warm-up lambda and the straight-through estimator
 * ([HF-1.58] "Dynamic warm-up quantization": lambda = min(step / total_steps, 1) scales
 * the difference between quantized and original values, x + lambda (Q(x) - x);
 * "Training with the straight-through estimator (STE)": the gradient of round() is
 * taken as 1, so a quantizer passes its output gradient to its input unchanged; "How
 * quantization works": quantized values are rescaled back, beta * q and Xq / s_t).
 * The matrix products of a training step around these (bf16 inputs, fp32 accumulation)
 * are plain GEMMs left to the caller's BLAS.
 *
 * bitlinear_warmup_lambda: min(step / total, 1) as fp32 (0 for step <= 0, 1 for
 * total <= 0). */
float bitlinear_warmup_lambda(int64_t step, int64_t total);

/* W_out[o, k] = bf16(w + lambda * (beta * q - w)), q the code of bitlinear_quantize_weights
 * for beta = w_scale[0] (so w_scale must come from that call on the same W); every
 * operation is one fp32 rounding, bf16 rounds to nearest even.
 *   W       device fp32 [N, K], 16-byte aligned;   w_scale device fp32 [1]
 *   lambda  in [0, 1];                             W_out   device bf16 bits [N, K], 16-byte aligned */
bl_status bitlinear_fake_quant_weights(const float* W, int64_t N, int64_t K, const float* w_scale,
                                       float lambda, uint16_t* W_out, bl_stream_t stream);

/* bitlinear_quantize_acts (same Xq, x_scale), plus
 *   X_out[t, k] = bf16(y + lambda * (Xq / s_t - y)), y the RMSNorm output (x with
 *                 BL_NO_NORM), Xq / s_t one fp32 division, every step one fp32 rounding
 *   x_rinv[t]   = r of the RMSNorm in fp64 (1 with BL_NO_NORM), or NULL
 *   X_out       device bf16 bits [T, K], 16-byte aligned; x_rinv 8-byte aligned */
bl_status bitlinear_fake_quant_acts(const float* X, const float* gain, int64_t T, int64_t K,
                                    float eps, uint32_t flags, float lambda, int8_t* Xq,
                                    float* x_scale, uint16_t* X_out, double* x_rinv,
                                    bl_stream_t stream);

/* Backward of y = x * r * g (r from x_rinv), the norm in front of the quantizer; the
 * quantizer's gradient is the identity, so dY is the gradient with respect to X_out:
 *   dX[t, k]  = fp32(r g_k dy_k - x_k r^3 (sum_j g_j dy_j x_j) / K), fp64 arithmetic
 *   dgain[k]  = fp32(sum_t r_t dy_tk x_tk) (fp64), when dgain is not NULL
 * gain NULL means unit gain. All arrays fp32 [T, K] / [K], 4-byte aligned. */
bl_status bitlinear_rmsnorm_backward(const float* X, const float* gain, const double* x_rinv,
                                     const float* dY, int64_t T, int64_t K, float* dX,
                                     float* dgain, bl_stream_t stream);

/* ---------------------------------------------------------------- BitDelta
 *
 * One base weight matrix shared by B fine-tuned models, each model stored as a 1-bit
 * delta ([BitDelta] "BitDelta: Your Fine-Tune May Only Be Worth One Bit": Eq. (1)
 * delta ~ alpha * Sign(delta), Eq. (2) Sign(W) = +1 for W > 0 and -1 otherwise, Eq. (4)
 * alpha = mean |delta|, Eq. (6) y_i = W_base x_i + alpha_i Sign(delta_i) x_i).
 * Shapes: W_base bf16 bits [N, M]; 1 <= B <= 8 models; M % 16 == 0, 16 <= M <= 8192,
 * N * M * 2 < 2^31 (else BL_ERR_DIM).
 * D (the batched deltas): uint8 [N, M], 16-byte aligned: row n, 16-code group j, model
 * slot i (of 8) at bytes ((n * M/16 + j) * 8 + i) * 2; bit c of the pair is code 16j + c,
 * set for +1; slots >= B are not read.
 *
 * bitlinear_bitdelta_compress: model `model`'s signs and scale from W_fine (fp32 [N, M],
 * 16-byte aligned): delta = fp32(W_fine - W_base); alpha[model] = fp32((exact sum of
 * |delta|, rounded once to fp64) / (N*M)); its bit pairs written into D (16-byte
 * aligned); other slots' bytes untouched. workspace as for bitlinear_quantize_weights. */
bl_status bitlinear_bitdelta_compress(const float* W_fine, const uint16_t* W_base, int64_t N,
                                      int64_t M, int B, int model, uint8_t* D, float* alpha,
                                      void* workspace, size_t workspace_bytes,
                                      bl_stream_t stream);

/* Y[i, n] = sum_k base[n, k] X[i, k] + alpha_i * sum_k c_i[n, k] X[i, k] for the B
 * tokens X fp32 [B, M] (16-byte aligned), Y fp32 [B, N]. fp32 arithmetic: the base part
 * with FMAs per 16 codes, the delta part as 2 * (sum of x where the bit is set) - sum x,
 * partial sums added across lanes and waves; the order of the final float additions
 * depends on scheduling, so the last bits of Y may vary from call to call. */
bl_status bitlinear_bitdelta_forward(const uint16_t* W_base, const uint8_t* D, const float* alpha,
                                     const float* X, int64_t N, int64_t M, int B, float* Y,
                                     bl_stream_t stream);

/* ---------------------------------------------------------------- rooflines
 *
 * The two rooflines the products are judged by, measured on the part itself
 * ([HF-1.58] "Tiled matrix multiplication": memory bandwidth and redundant accesses
 * bound the product, so a decode kernel is compared with a plain read of the same
 * bytes; the prefill GEMM with the matrix-core rate).
 *
 * bitlinear_roof_read: reads `count` (1..BL_MAX_GROUP) device buffers once (bytes[i]
 * a positive multiple of 16, bases 16-byte aligned), 16 bytes per lane and load, and
 * writes one word per wave to sink (device, BL_ROOF_READ_SINK_BYTES). schedule 0..3
 * picks how 1 KiB blocks map to waves (0: grid-stride, one block in flight per wave;
 * 1: grid-stride, two in flight; 2: a contiguous share per wave, two in flight; 3: as
 * 0 with no per-block buffer lookup, for one buffer, else as 0); the fastest, timed, is
 * the read roof of those buffers.
 *
 * bitlinear_roof_mfma_i8: `workgroups` workgroups of 4 waves each issue 8 * iters
 * v_mfma_i32_32x32x32_i8 (65536 int8 ops each) on register operands; sink (device int32,
 * workgroups * 256 entries) receives a checksum per lane, clocks (device uint64,
 * workgroups * 16 entries) per wave its start and end shader clock (s_memtime) and
 * start and end 100 MHz reference clock (s_memrealtime), in that order. */
#define BL_ROOF_READ_SINK_BYTES ((size_t)65536)
bl_status bitlinear_roof_read(const void* const* bufs, const int64_t* bytes, int count,
                              int schedule, uint32_t* sink, bl_stream_t stream);
bl_status bitlinear_roof_mfma_i8(int iters, int workgroups, int32_t* sink, uint64_t* clocks,
                                 bl_stream_t stream);

/* ---------------------------------------------------------------- misc */
const char* bitlinear_status_str(bl_status s);
/* Text of the last failing HIP call made by this thread ("" if none). */
const char* bitlinear_last_hip_error(void);
int bitlinear_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
