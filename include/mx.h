/*
 * mx.h -- C ABI of libmx.so: MX (microscaling) quantization and the
 * block-scaled low-precision GEMM on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited as [tag, section]):
 *   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
 *          (blog.zhiliyouxian.com)
 *   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践" (kongchang.com)
 *   [COAT] write-up of "COAT: Compressing Optimizer States and Activation
 *          for memory efficient FP8 Training" (dignews.cc)
 *   Element encodings and the shared-exponent rule: OCP Microscaling (MX)
 *   Formats specification v1.0.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates no memory and keeps no state between calls, with
 *     one exception: the 4 KiB per-GPU scratch array of
 *     mx_predict_tensor_scale_noalloc (see there).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only enqueues work on it and returns without synchronizing; outputs
 *     are valid once the stream reaches that point.
 *   - Arguments are validated on the host before any HIP call; on any
 *     error nothing is enqueued and the status says why.  No exceptions
 *     cross the ABI.  MX_ERR_HIP reports a failed launch (text via
 *     mx_last_error_message()).
 *   - Calls on different streams that write the same buffers race; calls
 *     on one stream are ordered.
 */
#ifndef MX_H
#define MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, bad shape */
    MX_ERR_UNSUPPORTED = 2,   /* a valid option this library does not build */
    MX_ERR_ALIGNMENT = 3,     /* pointer / leading dimension not 16-byte aligned */
    MX_ERR_HIP = 4            /* kernel launch failed */
} mx_status;

/* source dtype of the tensor being quantized */
enum { MX_SRC_F32 = 0, MX_SRC_BF16 = 1 };

/* element formats: FP8 E4M3 (max 448), FP8 E5M2 (max 57344), FP4 E2M1
 * (max 6; 1 sign, 2 exponent, 1 mantissa bit [FAF, "FP4加速为何常常纸上富贵"]) */
enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M1 = 2 };

/* scale formats: E8M0 power-of-two per 32-block only, or MOSS two-level:
 * an FP32 per-tensor scale amax/Fmax on top of the E8M0 block scales
 * ([MOSS, "创新 1：两级微缩放策略", "两级缩放实现"]) */
enum { MX_SCALE_E8M0 = 0, MX_SCALE_E8M0_TENSOR_F32 = 1 };

/* for the two-level format: compute the per-tensor scale from the tensor,
 * or read a caller-provided one (e.g. a predicted weight scale,
 * [MOSS, "创新 2：权重自动缩放"]) */
enum { MX_TSCALE_COMPUTE = 0, MX_TSCALE_PROVIDED = 1 };

/* rounding: round-to-nearest-even, or stochastic rounding driven by
 * Philox4x32-10 ([FAF, "两个关键的数值技巧"]) */
enum { MX_RNE = 0, MX_SR = 1 };

/* block axis / stored layout of a quantized copy:
 *   MX_AXIS_ROW: 1x32 blocks along each row; codes stored [rows][cols],
 *                scales [rows][cols/32]
 *   MX_AXIS_COL: 32x1 blocks down each column; the copy is stored
 *                TRANSPOSED: codes [cols][rows], scales [cols][rows/32]
 * FP4 codes are packed two per byte along the stored row, element 2j in
 * the low nibble of byte j.  Stored rows are dense (no padding). */
enum { MX_AXIS_ROW = 0, MX_AXIS_COL = 1 };

/* output dtype of mx_gemm / mx_dequantize */
enum { MX_OUT_F32 = 0, MX_OUT_BF16 = 1 };

typedef struct {
    int32_t fmt;        /* MX_E4M3 / MX_E5M2 / MX_E2M1 */
    int32_t block;      /* must be 32 */
    int32_t scale_fmt;  /* MX_SCALE_E8M0 / MX_SCALE_E8M0_TENSOR_F32 */
    int32_t tscale;     /* MX_TSCALE_COMPUTE / MX_TSCALE_PROVIDED (two-level only) */
    int32_t rounding;   /* MX_RNE / MX_SR */
    int32_t hadamard;   /* 1: fixed-sign 32-point Hadamard along the block axis first */
    uint64_t seed;      /* SR: Philox key = (seed low 32, seed high 32) */
    uint32_t offset;    /* SR: fourth Philox counter word */
    uint32_t reserved;  /* must be 0 */
} mx_qconfig;

/*
 * mx_quantize -- one quantized copy of a 2-D tensor.
 *
 * Per block of 32 elements along `axis` ([MOSS, "两级缩放实现"] for the
 * steps, [FAF, "两个关键的数值技巧"] for SR and the Hadamard):
 *   1. two-level only: s_t = amax(|x|)/Fmax (IEEE fp32 division; 1 if the
 *      tensor is all zero) and x <- x / s_t (IEEE fp32 division);
 *   2. if cfg->hadamard: v = H32 * block (unnormalised Sylvester FWHT in
 *      fp32, stages 1,2,4,8,16);
 *   3. e = floor(log2(max|v|)) - emax(fmt), clamped to [-127,127] (-127
 *      for an all-zero block); scale byte = e + 127; a block holding a
 *      NaN or Inf gets byte 0xFF and every element the code 0x7F (the
 *      format's NaN; E2M1, which has none: 0);
 *   4. y = v * 2^-e (exact); RNE, or SR: with lo <= |y| < hi the
 *      neighbouring codes and F = floor((|y|-lo)/(hi-lo) * 2^32), round up
 *      iff u < F, where u is word (idx & 3) of Philox4x32-10 with counter
 *      (idx>>2 low, idx>>2 high, axis, offset), key (seed low, seed high)
 *      and idx = r*cols + c the element's row-major index in the source;
 *      |y| >= Fmax saturates to +-Fmax; the sign is kept (also for zero).
 *
 * x:     source, `src_dtype`, rows x cols with row stride `ld` elements,
 *        ld >= cols, aligned to the element size.  (16-byte aligned x with
 *        ld*elem_size a multiple of 16 takes the vector-load path.)
 * rows, cols: > 0.  MX_AXIS_ROW needs cols % 32 == 0; MX_AXIS_COL needs
 *        rows % 32 == 0.
 * q, scales: the stored copy (layouts above); q 16-byte aligned.
 * tensor_scale: one fp32 in device memory.  Two-level + COMPUTE: written
 *        with s_t.  While the amax is reduced, the scale array (and, for a
 *        tiny tensor, this word) holds partial maxima, so neither may be
 *        read before the stream reaches the end of this call.
 *        Two-level + PROVIDED: read.  MX_SCALE_E8M0: ignored (may be NULL).
 * Errors: MX_ERR_INVALID_ARG (null pointers, block != 32, bad enum,
 *        reserved != 0, shapes above), MX_ERR_ALIGNMENT, MX_ERR_HIP.
 */
mx_status mx_quantize(const void* x, int32_t src_dtype, int64_t rows, int64_t cols, int64_t ld,
                      int32_t axis, const mx_qconfig* cfg, void* q, uint8_t* scales,
                      float* tensor_scale, void* stream);

/*
 * mx_quantize_dual_layout -- both copies from one read of the source
 * ([FAF, "格式感知融合的设计思路"]: the producer writes the layouts its
 * consumers take, with no separate re-layout pass).  Same arithmetic as
 * two mx_quantize calls (MX_AXIS_ROW into q_row/s_row, MX_AXIS_COL into
 * q_col/s_col) with the same cfg; SR draws the two copies from
 * independent streams (axis word 0 and 1).  Needs rows % 32 == 0 and
 * cols % 32 == 0.  Errors as mx_quantize.
 */
mx_status mx_quantize_dual_layout(const void* x, int32_t src_dtype, int64_t rows, int64_t cols,
                                  int64_t ld, const mx_qconfig* cfg, void* q_row,
                                  uint8_t* s_row, void* q_col, uint8_t* s_col,
                                  float* tensor_scale, void* stream);

/*
 * mx_gemm -- C = alpha' * A . B^T on scaled codes ([MOSS, "GEMM Kernel
 * 优化"]: the main loop multiplies codes with their block scales applied by
 * the matrix instruction; the per-tensor scales are applied once, in the
 * epilogue).
 *
 * qa, sa: A as written by the quantizer, [M][K] codes (K contiguous) and
 *         [M][K/32] E8M0 scales, element format fa.
 * qb, sb: B as [N][K] codes and [N][K/32] scales, element format fb.
 *         (A weight W[K][N] quantized with MX_AXIS_COL is exactly this.)
 * ta, tb: device fp32 per-tensor scales or NULL (= 1).
 * alpha' = alpha * ta * tb * (hadamard_k ? 1/32 : 1); set hadamard_k iff
 *         both operands were quantized with the Hadamard along K (H.H^T =
 *         32 I).  Accumulation is fp32.
 * c:      [M][N] with row stride ldc >= N elements, MX_OUT_F32 or
 *         MX_OUT_BF16 (round to nearest even).
 * Supported pairs: fa, fb both FP8 (E4M3/E5M2 in any combination) or
 *         both E2M1.  0 < M, N < 2^31 - 256 (and fewer than 2^31 output
 *         tiles of 256x256); 0 < K <= 2^23 and K % 32 == 0.
 * Errors: MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED (mixed FP8/FP4),
 *         MX_ERR_ALIGNMENT (qa, qb not 16-byte aligned), MX_ERR_HIP.
 */
mx_status mx_gemm(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                  const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                  int64_t M, int64_t N, int64_t K, float alpha, int32_t hadamard_k,
                  void* c, int32_t out_dtype, int64_t ldc, void* stream);

/*
 * mx_gemm_quantized -- mx_gemm whose epilogue writes C already MX-quantized
 * for the next layer ([FAF, "格式感知融合的设计思路"]: the producer emits
 * the layout and format its consumer reads, with no separate pass over a
 * bf16 C).  The fp32 value of each output is exactly the one mx_gemm
 * writes with MX_OUT_F32 (alpha' * accumulator, one fp32 multiply); those
 * values are then encoded as mx_quantize does for MX_AXIS_ROW with
 * MX_SCALE_E8M0 and MX_RNE: 1x32 blocks along each row of C, shared
 * exponent floor(log2 amax) - emax, saturating round-to-nearest-even.
 *
 * Operands, alpha, hadamard_k: as mx_gemm.
 * out_fmt: MX_E4M3 or MX_E5M2 (E2M1: MX_ERR_UNSUPPORTED).
 * qc:    [M][N] codes, dense (row stride N bytes), 16-byte aligned.
 * sc:    [M][N/32] E8M0 scale bytes.
 * Needs N % 32 == 0, and the operands in the form the fast GEMM kernel
 * takes: rows of K holding a multiple of 128 bytes of codes (FP8: K % 128
 * == 0; FP4: K % 256 == 0) and 4-byte aligned sa, sb (else
 * MX_ERR_UNSUPPORTED).  Other errors as mx_gemm.
 */
mx_status mx_gemm_quantized(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                            const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                            int64_t M, int64_t N, int64_t K, float alpha, int32_t hadamard_k,
                            int32_t out_fmt, void* qc, uint8_t* sc, void* stream);

/*
 * mx_dequantize -- inverse of mx_quantize ([MOSS, "两级缩放实现"]:
 * micro-scale first, then the tensor scale): per element
 * decode(code) * 2^(byte-127) (exact in fp32), then, if `hadamard`, the
 * inverse transform FWHT32(.) * 1/32 along the block, then, if
 * tensor_scale != NULL, one fp32 multiply by *tensor_scale.
 * q, scales: a copy in the stored layout of `axis` for a rows x cols source.
 * out: rows x cols in the SOURCE layout (row-major, dense), MX_OUT_F32 or
 *      MX_OUT_BF16.
 * Shapes as mx_quantize.  Errors: MX_ERR_INVALID_ARG, MX_ERR_ALIGNMENT
 * (q not 16-byte aligned), MX_ERR_HIP.
 */
mx_status mx_dequantize(const void* q, const uint8_t* scales, const float* tensor_scale,
                        int32_t fmt, int64_t rows, int64_t cols, int32_t axis, int32_t hadamard,
                        void* out, int32_t out_dtype, void* stream);

/*
 * mx_predict_tensor_scale -- MOSS weight auto-scaling ([MOSS, "创新 2：权重
 * 自动缩放"]): the per-tensor scale of the NEXT step's weights, predicted
 * from this step's weights W and update direction g without a pass over
 * the updated weights.  An update W' = W - lr*g moves no element by more
 * than lr*max|g|, so max|W'| <= max|W| + lr*max|g| (exactly, also in fp32
 * arithmetic: rounding is monotone), and
 *     scale_out = RN(RN(max|W| + RN(lr * max|g|)) / Fmax(fmt))
 * -- product, sum and IEEE division each rounded once, in that order
 * (the page's int8 illustration divides by 127; Fmax is 448 / 57344 / 6).
 * 1 when the sum is 0.  Non-finite inputs follow IEEE arithmetic: NaN
 * when W or g holds a NaN, and when lr == 0 and g holds an Inf (0 * Inf);
 * otherwise +Inf when W or g holds an Inf.  Pass the result to
 * mx_quantize / mx_quantize_dual_layout with
 * MX_SCALE_E8M0_TENSOR_F32 and MX_TSCALE_PROVIDED for W'.
 *
 * w, g:   device tensors of `src_dtype`, both rows x cols, row strides
 *         ld_w, ld_g >= cols elements, aligned to the element size.  g is
 *         the direction the step subtracts (the gradient for the page's
 *         W - lr*gradient form).
 * lr:     finite, >= 0.
 * work:   caller-owned device workspace of at least
 *         mx_predict_workspace_bytes() bytes, 4-byte aligned; it holds the
 *         partial maxima, and its contents are undefined afterwards.
 * scale_out: one fp32 in device memory, 4-byte aligned.
 * Errors: MX_ERR_INVALID_ARG (null pointers, bad dtype/format, shapes,
 *         lr, small workspace), MX_ERR_ALIGNMENT, MX_ERR_HIP.
 */
mx_status mx_predict_tensor_scale(const void* w, int64_t ld_w, const void* g, int64_t ld_g,
                                  int32_t src_dtype, int64_t rows, int64_t cols, float lr,
                                  int32_t fmt, void* work, int64_t work_bytes, float* scale_out,
                                  void* stream);

/* Bytes of workspace mx_predict_tensor_scale needs (a constant, 4096). */
int64_t mx_predict_workspace_bytes(void);

/*
 * mx_predict_tensor_scale_noalloc -- mx_predict_tensor_scale for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): no `work` argument, and
 * the call allocates nothing.  Same arguments (minus work / work_bytes),
 * result and errors as mx_predict_tensor_scale, computed by the same
 * kernels.
 *
 * The partial maxima go to a 4 KiB scratch array the library holds in each
 * GPU's memory from the first call on that GPU until the process ends (its
 * device address is looked up once per GPU).  Every input size fits it: at
 * most 512 partial maxima per tensor are kept whatever the shape, so no
 * size is rejected for the scratch.  Each call writes every scratch word it
 * then reads, so nothing needs clearing between calls, but all calls on one
 * GPU share the array: calls that overlap on one GPU (different streams,
 * or different host threads) race and must be ordered by the caller.
 * `stream` may belong to any GPU; the scratch of that GPU is used.
 */
mx_status mx_predict_tensor_scale_noalloc(const void* w, int64_t ld_w, const void* g, int64_t ld_g,
                                          int32_t src_dtype, int64_t rows, int64_t cols, float lr,
                                          int32_t fmt, float* scale_out, void* stream);

/*
 * mx_quantize_optstate -- FP8 optimizer states with dynamic range expansion
 * ([COAT, "解決方案：動態範圍擴充套件"]): each group of `group` consecutive
 * values of an fp32 optimizer state (e.g. Adam's first or second moment) is
 * expanded by f(x) = sign(x)|x|^k, with one k per group computed on the
 * fly, so that the group's max/min ratio matches the FP8 format's (Fmax /
 * smallest subnormal, about 2.3e5 for E4M3), then quantized.  Per group:
 *   amax = max|x|,  amin = smallest nonzero |x|,
 *   k = log2(Fmax / smallest subnormal) / log2(amax / amin)   (1 if amax == amin),
 *   q = RNE_saturating(sign(x) * (|x| / amax)^k * Fmax),
 * so the largest magnitude gets the format's top code and the smallest
 * nonzero one its smallest subnormal.  The page does not print f; the
 * COAT paper's form is used, normalised by amax (its per-group scale
 * amax^k / Fmax is then implicit).  Powers are exp2(k * log2(u)) with log2
 * and exp2 evaluated as a fixed sequence of fp32 operations (see
 * optstate.hip), so the codes depend only on IEEE fp32 arithmetic.
 * An all-zero group gets signed-zero codes, amax = k = 1; a group holding
 * a NaN or Inf gets the NaN code 0x7F everywhere and amax = k = NaN.
 *
 * x:      n fp32 values (device), 16-byte aligned; groups are consecutive.
 * n:      > 0, a multiple of group.
 * group:  32, 64, 128 or 256.
 * fmt:    MX_E4M3 or MX_E5M2 (MX_E2M1: MX_ERR_UNSUPPORTED).
 * q:      n codes, one byte each, 4-byte aligned.
 * amax, kexp: n / group fp32 each (the group's max |x| and k), 4-byte aligned.
 * Errors: MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_ALIGNMENT, MX_ERR_HIP.
 */
mx_status mx_quantize_optstate(const float* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q, float* amax,
                               float* kexp, void* stream);

/*
 * mx_dequantize_optstate -- the inverse: out = sign(q) * amax *
 * (|decode(q)| / Fmax)^(1/k), per element, with 1/k one fp32 division and
 * the power as in mx_quantize_optstate; NaN where the code, amax or k is NaN.
 * Arguments as mx_quantize_optstate; out: n fp32, 16-byte aligned.
 */
mx_status mx_dequantize_optstate(const uint8_t* q, const float* amax, const float* kexp, int64_t n, int32_t group,
                                 int32_t fmt, float* out, void* stream);

/*
 * mx_quantize_nvfp -- an NVFP4 copy of a matrix with its scale domain, for
 * the nvfp routes of [FAF, "格式感知融合的设计思路"] (each quantization
 * producer bound to its scale domain and its consumer's layout: global nvfp
 * and CTA-local nvfp beside native mxfp) and [FAF, "FP4加速为何常常纸上富贵"]
 * (nvfp: one scale per block).  The pages fix neither block size nor scale
 * format; NVIDIA's NVFP4 is used: E2M1 codes in blocks of 16 along the
 * stored row, an unsigned E4M3 scale per block, and an FP32 second-level
 * scale s = amax / (6 * 448) over the scale domain:
 *   local = 0 (global nvfp): one domain, the whole matrix (tscale[0]);
 *   local = 1 (CTA-local nvfp): one domain per panel of 32 stored rows
 *     (tscale[p] covers stored rows 32p .. 32p + 31), the rows one GEMM
 *     tile consumes, so no reduction crosses panels.
 * Per block of 16 (each step one fp32 rounding): den = 6 * s;
 * sb = E4M3_RNE_saturating(block amax / den); d = decode(sb) * s;
 * code_i = E2M1_RNE_saturating(x_i * (1 / d)).  s is 1 for an all-zero
 * domain, NaN for one holding a NaN or Inf; a zero block scale gives
 * signed-zero codes; a block holding a NaN or Inf, or in a NaN domain,
 * gets scale code 0x7F (E4M3 NaN) and zero codes.
 *
 * x, src_dtype, rows, cols, ld: as mx_quantize (row-major source).
 * axis:   MX_AXIS_ROW: stored rows are source rows (blocks along cols);
 *         MX_AXIS_COL: stored rows are source columns (the transposed
 *         copy, blocks along rows).  The blocked length L (cols or rows)
 *         must be a multiple of 16; SR is the other dimension.
 * q:      SR x L/2 bytes (two codes per byte, element 2j in the low
 *         nibble), 16-byte aligned.
 * scales: SR x L/16 E4M3 codes.
 * tscale: 1 fp32 (global) or ceil(SR / 32) fp32 (local), 4-byte aligned.
 * The global route runs three kernels (panel maxima, their reduction,
 * quantization) and uses q as its scratch between them; the local route
 * runs two.  Errors: MX_ERR_INVALID_ARG, MX_ERR_ALIGNMENT, MX_ERR_HIP.
 */
mx_status mx_quantize_nvfp(const void* x, int32_t src_dtype, int64_t rows, int64_t cols, int64_t ld,
                           int32_t axis, int32_t local, uint8_t* q, uint8_t* scales, float* tscale,
                           void* stream);

/*
 * mx_dequantize_nvfp -- out = RN(RN(e2m1(code) * e4m3(sb)) * s) per element
 * (the first product exact), written row-major [rows][cols] (leading
 * dimension cols) whichever axis the copy has.  Arguments as
 * mx_quantize_nvfp; out: fp32 (MX_OUT_F32) or bf16 (MX_OUT_BF16, round to
 * nearest even), aligned to its element size.
 */
mx_status mx_dequantize_nvfp(const uint8_t* q, const uint8_t* scales, const float* tscale, int64_t rows,
                             int64_t cols, int32_t axis, int32_t local, void* out, int32_t out_dtype,
                             void* stream);

/*
 * mx_gemm_nvfp -- the GEMM that consumes nvfp copies ([FAF,
 * "格式感知融合的设计思路"]: the consumer applies each producer's scale
 * domain):  C[i][j] = alpha * sA(i) * sB(j) * sum_k Ahat[i][k] Bhat[j][k],
 * with Ahat = e2m1(code) * e4m3(block scale) and sA(i) = ta[0] (local_a = 0)
 * or ta[i / 32] (local_a = 1); likewise B.  qa/sa: the row copy of A
 * [M][K] (mx_quantize_nvfp, MX_AXIS_ROW); qb/sb: the copy of B whose stored
 * rows are B's N columns ([N][K]: MX_AXIS_COL of a [K][N] matrix).
 * gfx950's block-scaled matrix instruction takes power-of-two scales per
 * 32, so the kernel dequantizes each stage exactly to f16 and multiplies
 * on the f16 matrix cores with fp32 accumulation; alpha * sA(i) * sB(j) is
 * one fp32 factor per output, applied once.
 * K: a multiple of 64, at most 2^24.  0 < M, N < 2^31 - 256, and fewer
 * than 2^31 output tiles of 256 x 256.  qa, qb 16-byte
 * aligned; sa, sb, ta, tb 4-byte aligned.  c: fp32 or bf16 (round to
 * nearest even), leading dimension ldc >= N.
 * Errors: MX_ERR_INVALID_ARG, MX_ERR_ALIGNMENT, MX_ERR_HIP.
 */
mx_status mx_gemm_nvfp(const uint8_t* qa, const uint8_t* sa, const float* ta, int32_t local_a,
                       const uint8_t* qb, const uint8_t* sb, const float* tb, int32_t local_b,
                       int64_t M, int64_t N, int64_t K, float alpha, void* c, int32_t out_dtype,
                       int64_t ldc, void* stream);

/* Static text for a status code. */
const char* mx_status_string(mx_status status);

/* Text of the last MX_ERR_HIP / validation failure on the calling thread
 * (empty string if none).  Valid until the next call on this thread. */
const char* mx_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* MX_H */
