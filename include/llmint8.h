/*
 * llmint8.h - C ABI of an MI355X (gfx950) library for the LLM.int8()
 * mixed-precision decomposition linear layer (the forward of an int8 linear
 * layer that replaces a 16-bit one).
 *
 * The method, as the sources describe it:
 *  - "Hugging Face Quantization with bitsandbytes: 4-bit & 8-bit Models
 *    Explained", section 2 "LLM.int8(): Quantizing Without Degrading Large
 *    Models": a few feature dimensions carry outliers of large magnitude; those
 *    are computed in 16-bit, the rest is multiplied in int8 and converted back
 *    to 16-bit at the end. Section 3: the outlier cutoff (default 6.0) applies
 *    to hidden-state values.
 *  - "bitsandbytes: GPU-Accelerated Inference and Training at Lower Bit
 *    Depths", section "How LLM.int8() quantizes weights and activations":
 *    vector-wise quantization; outliers go through a separate 16-bit product.
 *  - "bitsandbytes" (glossary), introduction: weights are quantized when the
 *    model loads, from the full-precision checkpoint.
 *
 * What the library computes (T rows, K input features, N output features):
 *   O      = { h : some |X[t,h]| >= threshold }            (fp32 compare)
 *   a[t]   = max_{k not in O} |X[t,k]|
 *   Xq     = rne(fl32(X * fl32(127/a[t]))), 0 on columns in O or when a[t]=0
 *   b[n]   = max_k |W[n,k]|,  Wq = rne(fl32(W * fl32(127/b[n])))
 *   C      = Xq . Wq^T                                      (int32, exact)
 *   Wd[n,j]= fp16(fl32(fl32(Wq[n,O_j] * b[n]) / 127))
 *   Y      = fp16( C * a[t] * b[n] / 127^2  +  X[:,O] . Wd^T )  (fp32 sums)
 * rne is round-half-to-even; fl32 an IEEE fp32 operation.
 *
 * Conventions for every entry point:
 *  - Matrices are dense and row-major (row stride = row length). Device
 *    pointers must be 16-byte aligned (sW, aX: 4-byte). fp16 data is IEEE
 *    binary16 passed as void*.
 *  - The caller owns every buffer. The library never allocates, frees or keeps
 *    a pointer past the call.
 *  - stream is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; outputs are valid once the stream has reached the call.
 *    No call synchronises the host or copies device data to the host.
 *  - Arguments are validated on the host before anything is enqueued. An
 *    error return means nothing was enqueued, except LLMINT8_ERR_HIP, which
 *    reports a failed launch (llmint8_last_hip_error() gives the HIP code).
 *  - Inputs must be finite. Non-finite inputs give unspecified results.
 *  - Calls that share a workspace must not run concurrently.
 */
#ifndef LLMINT8_H
#define LLMINT8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define LLMINT8_API __attribute__((visibility("default")))
#else
#define LLMINT8_API
#endif

typedef int llmint8_status;

#define LLMINT8_OK               0
#define LLMINT8_ERR_INVALID_ARG -1 /* null pointer, size <= 0 (T < 0), bad threshold, misaligned */
#define LLMINT8_ERR_UNSUPPORTED -2 /* K % 16 != 0, K > 65536, N*K or T*K >= 2^31 (backward: N % 8 != 0 or N > 65536) */
#define LLMINT8_ERR_WORKSPACE   -3 /* workspace smaller than llmint8_workspace_bytes_path(T,K,N,path) */
#define LLMINT8_ERR_HIP         -4 /* a HIP launch or runtime call failed */

/* Kernel route for llmint8_linear_debug / llmint8_linear_timed. */
#define LLMINT8_PATH_AUTO 0 /* what llmint8_linear uses */
#define LLMINT8_PATH_GEMM 1 /* scan + quantize + int8 MFMA GEMM (3 kernels), any T */
#define LLMINT8_PATH_GEMV 2 /* one fused weight-streaming kernel, small T only */
/* The GEMM route with a fixed output tile (N x T) instead of the one the
 * host's cost model picks: for tests and tuning, debug and timed calls only. */
#define LLMINT8_PATH_GEMM_256x256 16
#define LLMINT8_PATH_GEMM_192x256 17
#define LLMINT8_PATH_GEMM_256x128 18
#define LLMINT8_PATH_GEMM_128x128 19
#define LLMINT8_PATH_GEMM_352x256 20

/*
 * Vector-wise int8 quantization of a weight, done once when a layer is loaded
 * ("bitsandbytes" glossary, introduction; "bitsandbytes: GPU-Accelerated
 * Inference ...", "How LLM.int8() quantizes weights and activations").
 *   W   [in]  fp16 [N, K], device
 *   Wq  [out] int8 [N, K], device: rne(fl32(W[n,k] * fl32(127 / sW[n])))
 *   sW  [out] fp32 [N], device: row absmax max_k |W[n,k]| (0 for a zero row,
 *             whose codes are then all 0)
 * Requires N >= 1, 1 <= K, K % 16 == 0, N*K < 2^31.
 */
LLMINT8_API llmint8_status llmint8_quantize_weight(const void* W, int64_t N, int64_t K, int8_t* Wq,
                                       float* sW, void* stream);

/*
 * Bytes of device workspace llmint8_linear needs for a call with these sizes,
 * which never depends on the data. It is 0 when the call takes the fused
 * decode kernel (T <= llmint8_gemv_max_rows(K)), which keeps everything in
 * LDS. On the GEMM route it is the int8 activations (T*K bytes) and a few
 * small tables, plus room for the 16-bit operands of the first 512 outlier
 * columns (2*(T+N) bytes per column, at most 2*(T+N)*K for K < 512). A larger
 * workspace holds the operands of more outlier columns; the epilogue forms
 * those of columns past what the workspace holds from X and Wq directly, with
 * the same values, so any outlier count is handled. Returns 0 for invalid
 * sizes.
 */
LLMINT8_API size_t llmint8_workspace_bytes(int64_t T, int64_t K, int64_t N);

/*
 * llmint8_workspace_bytes for a debug or timed call with the given route
 * (LLMINT8_PATH_*): 0 for the fused decode route, the GEMM route's size for
 * the GEMM route at any T. Returns 0 for invalid sizes or an unknown path.
 */
LLMINT8_API size_t llmint8_workspace_bytes_path(int64_t T, int64_t K, int64_t N, int path);

/*
 * The forward of the LLM.int8() linear layer ("Hugging Face Quantization with
 * bitsandbytes ...", sections 2 and 3):
 *   X         [in]  fp16 [T, K], device (activations / hidden states)
 *   Wq, sW    [in]  from llmint8_quantize_weight (int8 [N, K], fp32 [N])
 *   threshold [in]  outlier cutoff on |x| (>= counts), > 0; +inf disables the
 *                   16-bit part; NaN or <= 0 is LLMINT8_ERR_INVALID_ARG
 *   Y         [out] fp16 [T, N], device
 *   workspace [tmp] device, >= llmint8_workspace_bytes(T, K, N) bytes,
 *                   256-byte aligned; contents on entry do not matter. May be
 *                   NULL (with any workspace_bytes) when that size is 0.
 * T == 0 is a valid no-op. The outlier set is decided over all T rows of the
 * call. Every stage runs on the GPU; the host never waits.
 */
LLMINT8_API llmint8_status llmint8_linear(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                              const float* sW, int64_t N, float threshold, void* Y,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * llmint8_linear with a chosen kernel route and copies of the intermediate
 * results, taken from the same kernels llmint8_linear runs. Every output
 * pointer below may be NULL (not written).
 *   path            LLMINT8_PATH_AUTO / _GEMM / _GEMV (GEMV needs
 *                   T <= llmint8_gemv_max_rows(K); else LLMINT8_ERR_UNSUPPORTED),
 *                   or LLMINT8_PATH_GEMM_<tile> (the GEMM route with that tile)
 *   outlier_bitmap  uint32 [ceil(K/32)]: bit h%32 of word h/32 set iff h in O
 *   outlier_idx     int32 [K]: ascending outlier columns in the first |O| slots
 *   outlier_count   int32 [1]: |O|
 *   Xq              int8 [T, K]
 *   aX              fp32 [T]: the row statistic a[t]
 *   C               int32 [T, N]: the int8 product before dequantization
 */
LLMINT8_API llmint8_status llmint8_linear_debug(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                    const float* sW, int64_t N, float threshold, void* Y,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int path, uint32_t* outlier_bitmap, int32_t* outlier_idx,
                                    int32_t* outlier_count, int8_t* Xq, float* aX, int32_t* C);

/*
 * llmint8_linear that also records caller-created HIP events (hipEvent_t
 * handles, passed as void*) on the stream around each kernel it launches:
 * events[0] before the first kernel, events[i+1] after kernel i. Needs
 * n_events >= kernels + 1 (at most 4); *kernels_launched (host int, may be
 * NULL) receives the kernel count. Used to time each kernel of a call.
 */
LLMINT8_API llmint8_status llmint8_linear_timed(const void* X, int64_t T, int64_t K, const int8_t* Wq,
                                    const float* sW, int64_t N, float threshold, void* Y,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    int path, void* const* events, int n_events,
                                    int* kernels_launched);

/*
 * Input gradient of the frozen layer, the step that lets an adapter be
 * trained on top of it ("Hugging Face Quantization with bitsandbytes ...",
 * the comparison table before section 1 and section 6: an int8 model is
 * frozen and an adapter is trained on top, with gradients flowing through the
 * quantized weights). The layer is taken as the linear map X -> X . Wdeq^T
 * with the stored weight dequantized for the operation ("bitsandbytes"
 * glossary, "Where it fits in the stack"):
 *   Wdeq[n,k] = fp16(fl32(fl32(Wq[n,k] * sW[n]) / 127))
 *   dX        = fp16( dY . Wdeq )            (fp16 products, fp32 sums)
 *
 *   dY        [in]  fp16 [T, N], device (gradient of the layer output)
 *   Wq, sW    [in]  from llmint8_quantize_weight (int8 [N, K], fp32 [N])
 *   dX        [out] fp16 [T, K], device
 *   workspace [tmp] not used: one kernel dequantizes Wq into the 16-bit
 *                   operand on the fly and keeps no copy of the weight
 *                   (llmint8_backward_workspace_bytes returns 0; any pointer,
 *                   NULL included, and size are accepted)
 * Requires, besides the forward's size limits, N % 8 == 0 and N <= 65536
 * (LLMINT8_ERR_UNSUPPORTED otherwise). T == 0 is a valid no-op. Results are
 * exact for the dequantization and within fp32 summation order for dX.
 */
LLMINT8_API size_t llmint8_backward_workspace_bytes(int64_t T, int64_t K, int64_t N);
LLMINT8_API llmint8_status llmint8_linear_backward_input(const void* dY, int64_t T, int64_t K,
                                                         const int8_t* Wq, const float* sW,
                                                         int64_t N, void* dX, void* workspace,
                                                         size_t workspace_bytes, void* stream);

/*
 * llmint8_linear_backward_input recording caller-created HIP events on the
 * stream: events[0] before its kernel, events[1] after it (n_events >= 2).
 * *kernels_launched (host int, may be NULL) receives 1.
 */
LLMINT8_API llmint8_status llmint8_linear_backward_input_timed(
    const void* dY, int64_t T, int64_t K, const int8_t* Wq, const float* sW, int64_t N, void* dX,
    void* workspace, size_t workspace_bytes, void* stream, void* const* events, int n_events,
    int* kernels_launched);

/*
 * The stored weight dequantized for an operation, transposed ("bitsandbytes"
 * glossary, "Where it fits in the stack"):
 *   WdT[k][n] = fp16(fl32(fl32(Wq[n,k] * sW[n]) / 127))
 *   Wq, sW [in]  from llmint8_quantize_weight (int8 [N, K], fp32 [N])
 *   WdT    [out] fp16 [K, N], device
 * Requires N % 8 == 0, N <= 65536 and the forward's limits on K and N*K. The result is
 * bit-exact for every sW that llmint8_quantize_weight produces.
 */
LLMINT8_API llmint8_status llmint8_dequantize_weight_t(const int8_t* Wq, const float* sW, int64_t N,
                                                       int64_t K, void* WdT, void* stream);

/*
 * The input gradient and the transposed dequantization in a chosen 16-bit
 * type (dtype LLMINT8_DTYPE_F16 or LLMINT8_DTYPE_BF16; constants below): dY,
 * WdT and dX are of that type, WdT = r16(fl32(fl32(Wq * b) / 127)) and
 * dX = r16(dY . Wdeq) with fp32 sums, r16 rounding to that type ("Hugging Face
 * Quantization with bitsandbytes ...", section 5: bfloat16 as the compute
 * type). Arguments, workspace and rules otherwise as for
 * llmint8_linear_backward_input / llmint8_dequantize_weight_t; an unknown
 * dtype is LLMINT8_ERR_INVALID_ARG.
 */
LLMINT8_API llmint8_status llmint8_linear_backward_input_ex(const void* dY, int dtype, int64_t T,
                                                            int64_t K, const int8_t* Wq,
                                                            const float* sW, int64_t N, void* dX,
                                                            void* workspace, size_t workspace_bytes,
                                                            void* stream);
LLMINT8_API llmint8_status llmint8_dequantize_weight_t_ex(const int8_t* Wq, const float* sW,
                                                          int64_t N, int64_t K, void* WdT,
                                                          int dtype, void* stream);

/* Element types: activations (the _ex entry points: F16 or BF16) and the
 * blockwise codec (F16 or F32). */
#define LLMINT8_DTYPE_F16  0 /* IEEE binary16 */
#define LLMINT8_DTYPE_F32  1 /* IEEE binary32 */
#define LLMINT8_DTYPE_BF16 2 /* bfloat16: the top 16 bits of an IEEE binary32 */

/*
 * Blockwise 8-bit codec ("bitsandbytes" glossary, "What it provides": a
 * tensor is quantized in blocks that each carry their own scaling factor, so
 * an outlier only affects its own block; "bitsandbytes: GPU-Accelerated
 * Inference and Training at Lower Bit Depths", 8-bit optimizers: block-wise
 * quantization of optimizer states). The flat tensor x of n elements is cut
 * into blocks of `block` consecutive elements (the last may be shorter):
 *   absmax[b] = max |x| over block b                       (fp32, exact)
 *   q[i]      = rne(fl32(x[i] * fl32(127 / absmax[b])))    (0 for a zero block)
 *   x'[i]     = fl32(fl32(q[i] * absmax[b]) / 127), rounded to dtype
 *   x, out  device, dtype LLMINT8_DTYPE_F16 or _F32, n elements, 16-byte aligned
 *   q       device int8 [n], 16-byte aligned
 *   absmax  device fp32 [ceil(n / block)]
 * Requires block a power of two in [64, 4096], n % 16 == 0 and n <= 2^30
 * (LLMINT8_ERR_UNSUPPORTED otherwise); n == 0 is a valid no-op. Inputs must be
 * finite. Results are bit-exact.
 */
LLMINT8_API llmint8_status llmint8_quantize_blockwise(const void* x, int dtype, int64_t n,
                                                      int64_t block, int8_t* q, float* absmax,
                                                      void* stream);
LLMINT8_API llmint8_status llmint8_dequantize_blockwise(const int8_t* q, const float* absmax,
                                                        int64_t n, int64_t block, void* out,
                                                        int dtype, void* stream);

/*
 * The entry points above for a chosen activation type and an optional bias
 * ("Hugging Face Quantization with bitsandbytes ...", section 5: storage type
 * and compute type are separate choices, bfloat16 preferred where the hardware
 * has it; "bitsandbytes: GPU-Accelerated Inference ...": Linear8bitLt replaces
 * a linear layer, which carries a bias).
 *   dtype  LLMINT8_DTYPE_F16 or LLMINT8_DTYPE_BF16: the type of W (for
 *          quantize_weight_ex), of X, bias and Y (for linear_ex). Every bf16
 *          value is exact in fp32, so the outlier test and the quantization
 *          are the same fp32 operations; with bf16 the outlier operand Wd is
 *          rounded to bf16, the 16-bit product takes bf16 operands and Y is
 *          rounded once to bf16 (nearest even).
 *   bias   device [N] in the activation type (2-byte aligned), or NULL; it is
 *          added to the fp32 sum before the single rounding of Y:
 *          Y = r16( C * a[t] * b[n] / 127^2 + X[:,O] . Wd^T + bias[n] )
 * Other arguments and rules as for llmint8_quantize_weight / llmint8_linear /
 * llmint8_linear_timed / llmint8_linear_debug; an unknown dtype is
 * LLMINT8_ERR_INVALID_ARG.
 */
LLMINT8_API llmint8_status llmint8_quantize_weight_ex(const void* W, int dtype, int64_t N, int64_t K,
                                                      int8_t* Wq, float* sW, void* stream);
LLMINT8_API llmint8_status llmint8_linear_ex(const void* X, int dtype, int64_t T, int64_t K,
                                             const int8_t* Wq, const float* sW, int64_t N,
                                             float threshold, const void* bias, void* Y,
                                             void* workspace, size_t workspace_bytes, void* stream);
LLMINT8_API llmint8_status llmint8_linear_timed_ex(const void* X, int dtype, int64_t T, int64_t K,
                                                   const int8_t* Wq, const float* sW, int64_t N,
                                                   float threshold, const void* bias, void* Y,
                                                   void* workspace, size_t workspace_bytes,
                                                   void* stream, int path, void* const* events,
                                                   int n_events, int* kernels_launched);
LLMINT8_API llmint8_status llmint8_linear_debug_ex(const void* X, int dtype, int64_t T, int64_t K,
                                                   const int8_t* Wq, const float* sW, int64_t N,
                                                   float threshold, const void* bias, void* Y,
                                                   void* workspace, size_t workspace_bytes,
                                                   void* stream, int path, uint32_t* outlier_bitmap,
                                                   int32_t* outlier_idx, int32_t* outlier_count,
                                                   int8_t* Xq, float* aX, int32_t* C);

/*
 * 4-bit weights: NF4 and FP4 ("bitsandbytes" glossary, "What it provides":
 * the 4-bit layer supports FP4 and NF4, quantizes the weight in blocks that
 * each carry a scaling factor and computes in FP16 or BF16 with the weight
 * dequantized per operation;
 * "Hugging Face Quantization with bitsandbytes ...", section 4: NF4 places its
 * levels where normally distributed weights concentrate, FP4 is a generic
 * 4-bit float).
 *
 * Code books (the pages name the types but print no values; this library
 * computes them on the host in binary64 and rounds once to fp32):
 *   NF4  the published NormalFloat construction (Dettmers et al., "QLoRA:
 *        Efficient Finetuning of Quantized LLMs", 2023, section 3): standard-normal quantiles at
 *        probabilities p_max + i (0.5 - p_max) / 8 (i = 0..7) above zero and
 *        their mirror images at p_max + i (0.5 - p_max) / 7 (i = 0..6) below,
 *        plus an exact zero, divided by the quantile at p_max = 1 - (1/32 +
 *        1/30) / 2; code c is the c-th level in ascending order (code 7 = 0).
 *   FP4  E2M1 (sign, two exponent bits with bias 1, one mantissa bit, exponent
 *        0 subnormal) divided by 6: code = 8 sign + magnitude bits, magnitudes
 *        {0, .5, 1, 1.5, 2, 3, 4, 6} / 6.
 * llmint8_code_book_4bit writes the 16 fp32 values, indexed by code, to the
 * host array `values`.
 *
 * Blockwise codes of a flat 16-bit tensor of n elements (a weight [N, K] is
 * taken row-major): block b is elements [b * block, (b + 1) * block);
 *   absmax[b] = max |w| over block b (fp32, exact)
 *   code      = the level nearest to fl32(w / absmax[b]) (0 when absmax is 0),
 *               decided against the fp32 midpoints fl32(fl32(l_i + l_{i+1}) *
 *               0.5) of adjacent distinct levels; a value on a midpoint takes
 *               the lower level; FP4 writes zero as +0
 *   packed    = two codes per byte, element 2 j in the low nibble of byte j
 *   Wdeq      = r16(fl32(value[code] * absmax[b])) in dtype (dequantize_4bit)
 * Arguments:
 *   W, out     device, dtype LLMINT8_DTYPE_F16 or _BF16, n elements, 16-byte aligned
 *   packed     device uint8 [n / 2], 16-byte aligned
 *   absmax     device fp32 [ceil(n / block)], 4-byte aligned
 *   quant_type LLMINT8_QUANT_NF4 or LLMINT8_QUANT_FP4 (else LLMINT8_ERR_INVALID_ARG)
 * Requires block a power of two in [64, 4096], n % 16 == 0 and n < 2^31
 * (LLMINT8_ERR_UNSUPPORTED otherwise); n == 0 is a no-op. Inputs must be
 * finite. Codes, absmax and Wdeq are bit-exact.
 *
 * llmint8_linear_4bit: Y = r16(X . Wdeq^T + bias), the decode-shaped forward
 * of a 4-bit layer, with the weight dequantized on the fly and never stored:
 *   X       device [T, K] in dtype, 16-byte aligned
 *   packed  device [N, K] codes (as above, n = N K), absmax per block
 *   bias    device [N] in dtype (2-byte aligned) or NULL
 *   Y       device [T, N] in dtype, 2-byte aligned
 * The products of the 16-bit operands are summed in fp32 and Y is rounded
 * once. Requires K % 128 == 0, N K < 2^31 and T K < 2^31
 * (LLMINT8_ERR_UNSUPPORTED); T == 0 is a no-op. Any T runs; the weight is read
 * once per 16 rows of X, so the route is meant for small T (decode).
 * All calls are asynchronous on `stream`, allocate nothing and use no workspace.
 */
#define LLMINT8_QUANT_NF4 0
#define LLMINT8_QUANT_FP4 1
LLMINT8_API llmint8_status llmint8_code_book_4bit(int quant_type, float* values);
LLMINT8_API llmint8_status llmint8_quantize_4bit(const void* W, int dtype, int64_t n, int64_t block,
                                                 int quant_type, uint8_t* packed, float* absmax,
                                                 void* stream);
LLMINT8_API llmint8_status llmint8_dequantize_4bit(const uint8_t* packed, const float* absmax,
                                                   int64_t n, int64_t block, int quant_type,
                                                   void* out, int dtype, void* stream);
LLMINT8_API llmint8_status llmint8_linear_4bit(const void* X, int dtype, int64_t T, int64_t K,
                                               const uint8_t* packed, const float* absmax,
                                               int64_t block, int quant_type, int64_t N,
                                               const void* bias, void* Y, void* stream);

/*
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops): llmint8_linear_ex without a
 * workspace argument, computing exactly what llmint8_linear_ex computes with
 * the same kernels. Its scratch is a static device array inside the library,
 * one per GPU, of llmint8_noalloc_scratch_bytes() bytes (64 MiB), held from
 * the first call on that GPU until the process ends; the call allocates
 * nothing. On the GEMM route it needs about T*K bytes plus 2*(T+N) bytes per
 * 32 outlier columns it holds (one chunk at least); a call whose shapes need
 * more returns LLMINT8_ERR_WORKSPACE before enqueuing anything. The fused
 * decode route (T <= llmint8_gemv_max_rows(K)) uses no scratch. All calls on
 * one GPU share its scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; calls in order on
 * one stream are safe. Arguments and errors otherwise as for
 * llmint8_linear_ex (HIP error of the one-time address lookup:
 * LLMINT8_ERR_HIP).
 */
LLMINT8_API llmint8_status llmint8_linear_noalloc(const void* X, int dtype, int64_t T, int64_t K,
                                                  const int8_t* Wq, const float* sW, int64_t N,
                                                  float threshold, const void* bias, void* Y,
                                                  void* stream);
LLMINT8_API size_t llmint8_noalloc_scratch_bytes(void);

/*
 * The GEMM tile the GEMM route picks for T rows and N output features on the
 * current device (its CU count; 256 when no device answers), as the
 * LLMINT8_PATH_GEMM_<tile> value that forces it; LLMINT8_ERR_INVALID_ARG for
 * T <= 0 or N <= 0. Host only; enqueues nothing.
 */
LLMINT8_API int llmint8_gemm_tile(int64_t T, int64_t N);

/* Largest T the fused GEMV route accepts for this K (0 if none). */
LLMINT8_API int llmint8_gemv_max_rows(int64_t K);

/* Static description of a status code. */
LLMINT8_API const char* llmint8_status_string(llmint8_status status);

/* HIP error code (hipError_t value) behind the last LLMINT8_ERR_HIP on this thread. */
LLMINT8_API int llmint8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LLMINT8_H */
