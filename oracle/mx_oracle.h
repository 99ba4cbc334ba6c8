/*
 * mx_oracle.h -- plain, slow CPU oracle for MX quantization and the
 * block-scaled GEMM.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the product library
 * never links, loads or calls it, and it shares no source with it.
 *
 * Sources (web pages; cited as [tag, section]):
 *   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
 *          (blog.zhiliyouxian.com)
 *   [COAT] write-up of "COAT: Compressing Optimizer States and Activation
 *          for memory efficient FP8 Training" (dignews.cc)
 *   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践" (kongchang.com)
 * Element formats and the shared-scale rule follow the OCP Microscaling
 * (MX) Formats specification v1.0, which the pages refer to by name but do
 * not restate.
 */
#ifndef MX_ORACLE_H
#define MX_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum { OR_E4M3 = 0, OR_E5M2 = 1, OR_E2M1 = 2 };
/* source dtypes */
enum { OR_SRC_F32 = 0, OR_SRC_BF16 = 1 };
/* block axis: ROW = 1x32 blocks along a row, copy stored [rows][cols];
 *             COL = 32x1 blocks down a column, copy stored [cols][rows] */
enum { OR_AXIS_ROW = 0, OR_AXIS_COL = 1 };

/* ---- formats ---- */
int      or_elem_bits(int fmt);                 /* 8 or 4 */
double   or_decode(int fmt, unsigned code);     /* exact value, NaN/Inf as such */
double   or_decode_e8m0(unsigned byte);         /* 2^(byte-127); NaN for 0xFF */
double   or_fmax(int fmt);                      /* largest finite magnitude */
int      or_emax(int fmt);                      /* exponent of or_fmax */
unsigned or_encode_rne(int fmt, double y);      /* saturating round-to-nearest-even */
unsigned or_encode_sr(int fmt, double y, uint32_t u); /* saturating stochastic rounding */
int      or_block_exponent(int fmt, double amax);     /* shared exponent e, -127..127 */
/* element-wise encode of n fp32 values (u ignored unless sr) -- for sweeps */
void     or_encode_array(int fmt, int sr, const float* y, const uint32_t* u, int64_t n,
                         uint8_t* out);

/* ---- helpers that the method is built from ---- */
void  or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void  or_fwht32(float v[32]);
float or_tensor_amax(const void* x, int src, int64_t rows, int64_t cols, int64_t ld);
float or_tensor_scale(int fmt, float amax);
double or_round_bf16(double x);
/* weight auto-scaling: predicted max|W - lr*g| bound and the scale from it */
float or_predict_max(const void* w, const void* g, int src, int64_t rows, int64_t cols,
                     int64_t ld_w, int64_t ld_g, float lr);
float or_predict_tensor_scale(const void* w, const void* g, int src, int64_t rows, int64_t cols,
                              int64_t ld_w, int64_t ld_g, float lr, int fmt);

/* ---- one block ----
 * v: the 32 values of the block after the optional two-level division and
 * Hadamard; u: one 32-bit random word per element (ignored for RNE).
 * codes get one code per element (unpacked, sign in the top bit of the
 * format's width); returns the E8M0 scale byte. */
unsigned or_quantize_block(int fmt, int sr, const float v[32], const uint32_t u[32],
                           uint8_t codes[32]);

/* ---- whole tensors ----
 * cfg_two_level: 0 = E8M0 only; 1 = FP32 per-tensor scale computed from the
 *   tensor (written to *tensor_scale); 2 = FP32 per-tensor scale read from
 *   *tensor_scale.
 * Outputs (packed; FP4 puts element 2j in the low nibble of byte j):
 *   axis ROW: q[rows][cols*bits/8], scales[rows][cols/32]
 *   axis COL: q[cols][rows*bits/8], scales[cols][rows/32]
 * Returns 0 on success, -1 on a shape the method does not define. */
int or_quantize(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis,
                int fmt, int two_level, int sr, int hadamard, uint64_t seed, uint32_t offset,
                uint8_t* q, uint8_t* scales, float* tensor_scale, int nthreads);

/* Quantize only the listed blocks.  Block b starts at source element
 * (r0[b], c0[b]) and runs along `axis`.  codes: [n][32] unpacked codes,
 * scales: [n].  s_t is the per-tensor scale to divide by (two_level != 0). */
int or_quantize_blocks(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis,
                       int fmt, int two_level, float s_t, int sr, int hadamard,
                       uint64_t seed, uint32_t offset, const int64_t* r0, const int64_t* c0,
                       int64_t n, uint8_t* codes, uint8_t* scales);

/* Inverse of or_quantize: out[rows][cols] (source layout), fp32. */
int or_dequantize(const uint8_t* q, const uint8_t* scales, const float* tensor_scale,
                  int fmt, int64_t rows, int64_t cols, int axis, int hadamard, float* out,
                  int nthreads);

/* C[i][j] = alpha' * sum_k Ahat[i][k] * Bhat[j][k] in double, with
 * alpha' = alpha * sA * sB * (hadamard_k ? 1/32 : 1); A is [M][K], B is [N][K]
 * (codes packed as or_quantize writes them, scales [rows][K/32]).
 * bound[i][j] = |alpha'| * sum_k |Ahat[i][k]| |Bhat[j][k]|.  ta/tb may be NULL. */
int or_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int fa,
            const uint8_t* qb, const uint8_t* sb, const float* tb, int fb,
            int64_t M, int64_t N, int64_t K, double alpha, int hadamard_k,
            double* C, double* bound, int nthreads);

/* Same, for the n listed output entries (ii[t], jj[t]). */
int or_gemm_entries(const uint8_t* qa, const uint8_t* sa, const float* ta, int fa,
                    const uint8_t* qb, const uint8_t* sb, const float* tb, int fb,
                    int64_t M, int64_t N, int64_t K, double alpha, int hadamard_k,
                    const int64_t* ii, const int64_t* jj, int64_t n,
                    double* C, double* bound, int nthreads);

/* ---- FP8 optimizer states with dynamic range expansion [COAT] ----
 * Groups of `group` consecutive fp32 values; per group amax and the
 * expansion exponent k; codes one byte per element (E4M3 or E5M2).
 * Returns 0, or -1 on bad arguments. */
float or_log2_fp32(float x);                 /* fixed fp32 evaluation, x > 0 */
float or_exp2_fp32(float y);
float or_pow_fp32(float u, float k);         /* u^k, u >= 0 */
int or_optstate_quantize(const float* x, int64_t n, int64_t group, int fmt, uint8_t* q, float* amax,
                         float* kexp, int nthreads);
int or_optstate_dequantize(const uint8_t* q, const float* amax, const float* kexp, int64_t n, int64_t group,
                           int fmt, float* out, int nthreads);

/* ---- nvfp routes [FAF] (reading: NVFP4, blocks of 16, E4M3 scales) ----
 * local = 0: one FP32 second-level scale (global); 1: one per 32 stored
 * rows.  Copies stored as mx: axis ROW [rows][cols/2] bytes, COL
 * [cols][rows/2]; block scales [stored rows][row length / 16]; tscale
 * [1] or [ceil(stored rows / 32)].  Returns 0, or -1 on bad shapes. */
int or_nvfp_quantize(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis, int local,
                     uint8_t* q, uint8_t* s16, float* tscale, int nthreads);
int or_nvfp_dequantize(const uint8_t* q, const uint8_t* s16, const float* tscale, int64_t rows, int64_t cols,
                       int axis, int local, float* out);
int or_nvfp_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int local_a,
                 const uint8_t* qb, const uint8_t* sb, const float* tb, int local_b,
                 int64_t M, int64_t N, int64_t K, double alpha, double* C, double* bound, int nthreads);
int or_nvfp_gemm_entries(const uint8_t* qa, const uint8_t* sa, const float* ta, int local_a,
                         const uint8_t* qb, const uint8_t* sb, const float* tb, int local_b,
                         int64_t M, int64_t N, int64_t K, double alpha, const int64_t* ii, const int64_t* jj,
                         int64_t n, double* C, double* bound, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
