/*
 * mx_oracle.c -- plain, slow, scalar CPU oracle.  TEST INFRASTRUCTURE:
 * used only by the tests, the smoke check and the CPU-baseline leg of the
 * benchmark.  Shares no source with the HIP library.
 *
 * Sources (web pages; cited as [tag, section]):
 *   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
 *          (blog.zhiliyouxian.com)
 *   [COAT] write-up of "COAT: Compressing Optimizer States and Activation
 *          for memory efficient FP8 Training" (dignews.cc)
 *   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践" (kongchang.com)
 *   OCP Microscaling (MX) Formats specification v1.0 for the element
 *   encodings and the shared-exponent rule (the pages name the MX standard
 *   but do not restate it).
 *
 * Style: every step is written the plain way -- values are held exactly in
 * double where the method treats them as exact reals, rounding is decided
 * by comparing against the enumerated code values, and there is no
 * blocking, vectorisation or reordering beyond what the method states.
 * Threads only split independent blocks / output rows.
 *
 * Parity pins: every function here is pinned by a CPU test (formats vs the
 * enumerated code sets, torch's float8 casts and the pages' constants;
 * shared exponent vs hand cases; Philox vs rocRAND's Philox4x32-10 engine;
 * FWHT vs scipy's Hadamard matrix; SR vs its expectation; GEMM vs a float64
 * library matmul and exact integer cases).  None is "parity unpinned".
 */
#include "mx_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element formats (OCP MX v1.0; E2M1's 1/2/1 bit split is also stated on
 * [FAF, "FP4加速为何常常纸上富贵"]; E4M3's 448 maximum and 0.00195 minimum
 * subnormal on [COAT, "FP8最佳化器狀態"] and [MOSS, "两级缩放实现"]).      */
/* ------------------------------------------------------------------ */

static int fmt_ebits(int fmt) { return fmt == OR_E4M3 ? 4 : fmt == OR_E5M2 ? 5 : 2; }
static int fmt_mbits(int fmt) { return fmt == OR_E4M3 ? 3 : fmt == OR_E5M2 ? 2 : 1; }
static int fmt_bias(int fmt) { return fmt == OR_E4M3 ? 7 : fmt == OR_E5M2 ? 15 : 1; }

int or_elem_bits(int fmt) { return 1 + fmt_ebits(fmt) + fmt_mbits(fmt); }

double or_decode(int fmt, unsigned code)
{
    const int E = fmt_ebits(fmt), M = fmt_mbits(fmt), B = fmt_bias(fmt);
    code &= (1u << (1 + E + M)) - 1u;
    const unsigned s = code >> (E + M);
    const unsigned e = (code >> M) & ((1u << E) - 1u);
    const unsigned m = code & ((1u << M) - 1u);
    const double sign = s ? -1.0 : 1.0;
    if (fmt == OR_E4M3 && e == 15 && m == 7) return NAN;          /* S.1111.111 */
    if (fmt == OR_E5M2 && e == 31) return m == 0 ? sign * INFINITY : NAN;
    if (e == 0) return sign * ldexp((double)m, 1 - B - M);        /* subnormal */
    return sign * ldexp(1.0 + (double)m / (double)(1u << M), (int)e - B);
}

double or_decode_e8m0(unsigned byte)
{
    byte &= 0xFFu;
    if (byte == 0xFFu) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* The positive finite magnitudes of a format, in code order: t[k] is the
 * value of code k (sign bit clear).  Built from or_decode, never typed in. */
typedef struct { int n; double t[128]; } mag_table;
static mag_table g_tab[3];
static pthread_once_t g_tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (int fmt = 0; fmt < 3; fmt++) {
        const unsigned ncodes = 1u << (or_elem_bits(fmt) - 1);   /* sign clear */
        int n = 0;
        for (unsigned k = 0; k < ncodes; k++) {
            double v = or_decode(fmt, k);
            if (!isfinite(v)) break;                             /* NaN / Inf at the top */
            g_tab[fmt].t[n++] = v;
        }
        g_tab[fmt].n = n;
    }
}

static const mag_table* table(int fmt)
{
    pthread_once(&g_tab_once, build_tables);
    return &g_tab[fmt];
}

double or_fmax(int fmt) { const mag_table* T = table(fmt); return T->t[T->n - 1]; }
int or_emax(int fmt) { return ilogb(or_fmax(fmt)); }

static unsigned nan_code(int fmt, int negative)
{
    /* FP8 formats: the all-ones magnitude 0x7F is a NaN in E4M3 and E5M2.
     * E2M1 has no NaN: such elements are written as +0 (their block's
     * scale byte 0xFF already marks the block as NaN).  The sign is not
     * used: IEEE 754 leaves the sign of a NaN produced by arithmetic (for
     * instance by the Hadamard) unspecified, so the code must not carry it. */
    (void)negative;
    if (fmt == OR_E2M1) return 0u;
    return 0x7Fu;
}

/* index i with t[i] <= a < t[i+1]; requires 0 <= a < fmax */
static int bracket(const mag_table* T, double a)
{
    int i = 0;
    while (T->t[i + 1] <= a) i++;
    return i;
}

unsigned or_encode_rne(int fmt, double y)
{
    const mag_table* T = table(fmt);
    const unsigned sign = signbit(y) ? 1u << (or_elem_bits(fmt) - 1) : 0u;
    if (isnan(y)) return nan_code(fmt, signbit(y) != 0);
    const double a = fabs(y);
    if (a >= T->t[T->n - 1]) return sign | (unsigned)(T->n - 1);   /* saturate */
    const int i = bracket(T, a);
    const double mid = 0.5 * (T->t[i] + T->t[i + 1]);              /* exact */
    int k;
    if (a < mid) k = i;
    else if (a > mid) k = i + 1;
    else k = (i % 2 == 0) ? i : i + 1;                              /* tie: even code */
    return sign | (unsigned)k;
}

unsigned or_encode_sr(int fmt, double y, uint32_t u)
{
    /* [FAF, "两个关键的数值技巧"]: round up or down with a probability that
     * follows the distance to the two neighbours, unbiased in expectation.
     * Bit-level reading: with F = floor(frac * 2^32), round up iff u < F. */
    const mag_table* T = table(fmt);
    const unsigned sign = signbit(y) ? 1u << (or_elem_bits(fmt) - 1) : 0u;
    if (isnan(y)) return nan_code(fmt, signbit(y) != 0);
    const double a = fabs(y);
    if (a >= T->t[T->n - 1]) return sign | (unsigned)(T->n - 1);
    const int i = bracket(T, a);
    const double frac = (a - T->t[i]) / (T->t[i + 1] - T->t[i]);    /* exact */
    const double F = floor(ldexp(frac, 32));
    const int k = ((double)u < F) ? i + 1 : i;
    return sign | (unsigned)k;
}

void or_encode_array(int fmt, int sr, const float* y, const uint32_t* u, int64_t n,
                     uint8_t* out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (uint8_t)(sr ? or_encode_sr(fmt, (double)y[i], u[i])
                              : or_encode_rne(fmt, (double)y[i]));
}

int or_block_exponent(int fmt, double amax)
{
    /* OCP MX: shared exponent = floor(log2(amax)) - emax(element format),
     * kept inside E8M0's range.  The power-of-two form is what makes the
     * dequantization exact ([MOSS, "Power-of-Two 的关键优势"]). */
    if (!(amax > 0.0)) return -127;
    int e = ilogb(amax) - or_emax(fmt);
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:   */
/* As Easy as 1, 2, 3", SC'11): 10 rounds of the 4x32 Philox S-box with   */
/* a Weyl-sequence key schedule.                                          */
/* ------------------------------------------------------------------ */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ------------------------------------------------------------------ */
/* 32-point Hadamard with fixed signs ([FAF, "两个关键的数值技巧"]):        */
/* Sylvester order H[i][j] = (-1)^popcount(i&j), unnormalised, computed   */
/* as a fast Walsh-Hadamard transform in fp32 with stages h=1,2,4,8,16.  */
/* ------------------------------------------------------------------ */
void or_fwht32(float v[32])
{
    for (int h = 1; h < 32; h <<= 1)
        for (int i = 0; i < 32; i++)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* ------------------------------------------------------------------ */
/* Two-level scaling ([MOSS, "两级缩放实现"]): level 1 is an FP32 per-     */
/* tensor scale amax / Fmax, and the tensor is divided by it.            */
/* ------------------------------------------------------------------ */
static float load_src(const void* x, int src, int64_t idx)
{
    if (src == OR_SRC_F32) return ((const float*)x)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16;   /* bf16 -> fp32, exact */
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

float or_tensor_amax(const void* x, int src, int64_t rows, int64_t cols, int64_t ld)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            const float a = fabsf(load_src(x, src, r * ld + c));
            if (isnan(a)) return NAN;
            if (a > amax) amax = a;
        }
    return amax;
}

float or_tensor_scale(int fmt, float amax)
{
    if (isnan(amax)) return NAN;
    if (amax == 0.0f) return 1.0f;             /* all-zero tensor: unit scale */
    const float fmax = (float)or_fmax(fmt);    /* 448, 57344 or 6: exact in fp32 */
    return amax / fmax;                        /* one IEEE binary32 division */
}

/* [MOSS, "创新 2：权重自动缩放"]: an update W' = W - lr*g moves no element
 * by more than lr*max|g|, so max|W'| <= max|W| + lr*max|g|.  The predicted
 * max is that sum, in fp32 as written: one product, then one sum (no fused
 * multiply-add); NaN if either tensor holds a NaN. */
float or_predict_max(const void* w, const void* g, int src, int64_t rows, int64_t cols,
                     int64_t ld_w, int64_t ld_g, float lr)
{
    const float aw = or_tensor_amax(w, src, rows, cols, ld_w);
    const float ag = or_tensor_amax(g, src, rows, cols, ld_g);
    if (isnan(aw) || isnan(ag)) return NAN;
    const float step = lr * ag;
    return aw + step;
}

/* the per-tensor scale of the next step's weights: predicted max / Fmax,
 * the same division (and the same unit scale for zero) as a computed
 * two-level scale.  The page divides by 127 for its int8 illustration;
 * Fmax of the element format is the FP8/FP4 reading. */
float or_predict_tensor_scale(const void* w, const void* g, int src, int64_t rows, int64_t cols,
                              int64_t ld_w, int64_t ld_g, float lr, int fmt)
{
    return or_tensor_scale(fmt, or_predict_max(w, g, src, rows, cols, ld_w, ld_g, lr));
}

double or_round_bf16(double x)
{
    /* nearest bfloat16 (8 significant bits, fp32 exponent range), ties to
     * even; overflow to +-inf */
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    const double a = fabs(x);
    int e = ilogb(a);
    if (e < -126) e = -126;                    /* bf16 subnormal spacing 2^-133 */
    const double q = ldexp(1.0, e - 7);
    const double lo = floor(a / q) * q, hi = lo + q;
    double r;
    if (a - lo < hi - a) r = lo;
    else if (a - lo > hi - a) r = hi;
    else r = (fmod(lo / q, 2.0) == 0.0) ? lo : hi;
    if (r > ldexp(255.0 / 128.0, 127)) r = INFINITY;   /* beyond the largest bf16 */
    return x < 0 ? -r : r;
}

/* ------------------------------------------------------------------ */
/* One block: amax -> E8M0 -> scale -> round -> code                      */
/* ------------------------------------------------------------------ */
unsigned or_quantize_block(int fmt, int sr, const float v[32], const uint32_t u[32],
                           uint8_t codes[32])
{
    int nonfinite = 0;
    double amax = 0.0;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(v[i])) nonfinite = 1;
        else if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
    }
    if (nonfinite) {                          /* NaN shared scale marks the block */
        for (int i = 0; i < 32; i++) codes[i] = (uint8_t)nan_code(fmt, signbit(v[i]) != 0);
        return 0xFFu;
    }
    const int e = or_block_exponent(fmt, amax);
    for (int i = 0; i < 32; i++) {
        const double y = ldexp((double)v[i], -e);   /* exact real */
        codes[i] = (uint8_t)(sr ? or_encode_sr(fmt, y, u[i]) : or_encode_rne(fmt, y));
    }
    return (unsigned)(e + 127);
}

/* the 32 source positions of a block, the values after level-1 scaling
 * and the optional Hadamard, and the per-element random words */
static void gather_block(const void* x, int src, int64_t cols, int64_t ld, int axis,
                         int two_level, float s_t, int sr, int hadamard, uint64_t seed,
                         uint32_t offset, int64_t r0, int64_t c0, float v[32], uint32_t u[32])
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int i = 0; i < 32; i++) {
        const int64_t r = axis == OR_AXIS_ROW ? r0 : r0 + i;
        const int64_t c = axis == OR_AXIS_ROW ? c0 + i : c0;
        float xv = load_src(x, src, r * ld + c);
        if (two_level) xv = xv / s_t;
        v[i] = xv;
        u[i] = 0;
        if (sr) {
            /* counter = (idx/4 low, idx/4 high, axis, offset) with idx the
             * element's row-major index in the source tensor */
            const uint64_t idx = (uint64_t)r * (uint64_t)cols + (uint64_t)c;
            const uint64_t n = idx >> 2;
            const uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), (uint32_t)axis, offset};
            uint32_t out[4];
            or_philox4x32_10(ctr, key, out);
            u[i] = out[idx & 3];
        }
    }
    if (hadamard) or_fwht32(v);
}

static void put_code(uint8_t* q, int bits, int64_t row_bytes, int64_t orow, int64_t ocol,
                     unsigned code)
{
    if (bits == 8) {
        q[orow * row_bytes + ocol] = (uint8_t)code;
    } else {
        uint8_t* p = &q[orow * row_bytes + ocol / 2];
        if (ocol % 2 == 0) *p = (uint8_t)((*p & 0xF0u) | (code & 0xFu));
        else *p = (uint8_t)((*p & 0x0Fu) | ((code & 0xFu) << 4));
    }
}

static unsigned get_code(const uint8_t* q, int bits, int64_t row_bytes, int64_t orow,
                         int64_t ocol)
{
    if (bits == 8) return q[orow * row_bytes + ocol];
    const uint8_t b = q[orow * row_bytes + ocol / 2];
    return ocol % 2 == 0 ? (b & 0xFu) : (b >> 4);
}

/* ------------------------------------------------------------------ */
/* tiny thread pool: run body(lo, hi, arg) on nthreads contiguous ranges */
/* ------------------------------------------------------------------ */
typedef void (*range_fn)(int64_t lo, int64_t hi, void* arg);
typedef struct { range_fn f; int64_t lo, hi; void* arg; } range_job;

static void* range_thread(void* p)
{
    range_job* j = (range_job*)p;
    j->f(j->lo, j->hi, j->arg);
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn f, void* arg)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
    if (nthreads == 1) { f(0, n, arg); return; }
    pthread_t th[256];
    range_job jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t].f = f;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
        jobs[t].arg = arg;
        pthread_create(&th[t], NULL, range_thread, &jobs[t]);
    }
    for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* Whole-tensor quantization                                             */
/* ------------------------------------------------------------------ */
typedef struct {
    const void* x; int src; int64_t rows, cols, ld; int axis, fmt, two_level; float s_t;
    int sr, hadamard; uint64_t seed; uint32_t offset; uint8_t* q; uint8_t* scales;
} quant_job;

static void quant_range(int64_t lo, int64_t hi, void* arg)
{
    const quant_job* J = (const quant_job*)arg;
    const int bits = or_elem_bits(J->fmt);
    /* the stored copy: ROW -> [rows][cols], COL -> [cols][rows] */
    const int64_t out_rows = J->axis == OR_AXIS_ROW ? J->rows : J->cols;
    const int64_t out_cols = J->axis == OR_AXIS_ROW ? J->cols : J->rows;
    const int64_t row_bytes = out_cols * bits / 8;
    const int64_t nblk = out_cols / 32;
    (void)out_rows;
    for (int64_t b = lo; b < hi; b++) {
        const int64_t orow = b / nblk, oblk = b % nblk;
        const int64_t r0 = J->axis == OR_AXIS_ROW ? orow : oblk * 32;
        const int64_t c0 = J->axis == OR_AXIS_ROW ? oblk * 32 : orow;
        float v[32];
        uint32_t u[32];
        uint8_t codes[32];
        gather_block(J->x, J->src, J->cols, J->ld, J->axis, J->two_level != 0, J->s_t, J->sr,
                     J->hadamard, J->seed, J->offset, r0, c0, v, u);
        J->scales[orow * nblk + oblk] = (uint8_t)or_quantize_block(J->fmt, J->sr, v, u, codes);
        for (int i = 0; i < 32; i++) put_code(J->q, bits, row_bytes, orow, oblk * 32 + i, codes[i]);
    }
}

static int shape_ok(int64_t rows, int64_t cols, int64_t ld, int axis)
{
    if (rows <= 0 || cols <= 0 || ld < cols) return 0;
    if (axis == OR_AXIS_ROW && cols % 32 != 0) return 0;
    if (axis == OR_AXIS_COL && rows % 32 != 0) return 0;
    return 1;
}

int or_quantize(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis,
                int fmt, int two_level, int sr, int hadamard, uint64_t seed, uint32_t offset,
                uint8_t* q, uint8_t* scales, float* tensor_scale, int nthreads)
{
    if (!shape_ok(rows, cols, ld, axis)) return -1;
    float s_t = 1.0f;
    if (two_level == 1) {
        s_t = or_tensor_scale(fmt, or_tensor_amax(x, src, rows, cols, ld));
        *tensor_scale = s_t;
    } else if (two_level == 2) {
        s_t = *tensor_scale;
    }
    quant_job J = {x, src, rows, cols, ld, axis, fmt, two_level, s_t, sr, hadamard,
                   seed, offset, q, scales};
    const int64_t nblocks = rows * cols / 32;
    parallel_for(nblocks, nthreads, quant_range, &J);
    return 0;
}

int or_quantize_blocks(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis,
                       int fmt, int two_level, float s_t, int sr, int hadamard,
                       uint64_t seed, uint32_t offset, const int64_t* r0, const int64_t* c0,
                       int64_t n, uint8_t* codes, uint8_t* scales)
{
    if (!shape_ok(rows, cols, ld, axis)) return -1;
    for (int64_t b = 0; b < n; b++) {
        const int64_t rr = r0[b], cc = c0[b];
        if (rr < 0 || cc < 0) return -1;
        if (axis == OR_AXIS_ROW && (rr >= rows || cc % 32 != 0 || cc + 32 > cols)) return -1;
        if (axis == OR_AXIS_COL && (cc >= cols || rr % 32 != 0 || rr + 32 > rows)) return -1;
        float v[32];
        uint32_t u[32];
        gather_block(x, src, cols, ld, axis, two_level != 0, s_t, sr, hadamard, seed, offset,
                     rr, cc, v, u);
        scales[b] = (uint8_t)or_quantize_block(fmt, sr, v, u, &codes[b * 32]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantization ([MOSS, "两级缩放实现"]: micro-scale first, then the      */
/* tensor scale).  Reading: undo in reverse order of quantization --     */
/* decode * 2^(byte-127) (exact), inverse Hadamard H/32, then * s_t.     */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint8_t* q; const uint8_t* scales; const float* ts; int fmt;
    int64_t rows, cols; int axis, hadamard; float* out;
} dq_job;

static void dq_range(int64_t lo, int64_t hi, void* arg)
{
    const dq_job* J = (const dq_job*)arg;
    const int bits = or_elem_bits(J->fmt);
    const int64_t out_cols = J->axis == OR_AXIS_ROW ? J->cols : J->rows;
    const int64_t row_bytes = out_cols * bits / 8;
    const int64_t nblk = out_cols / 32;
    for (int64_t b = lo; b < hi; b++) {
        const int64_t orow = b / nblk, oblk = b % nblk;
        const double s = or_decode_e8m0(J->scales[orow * nblk + oblk]);
        float v[32];
        for (int i = 0; i < 32; i++)
            v[i] = (float)(or_decode(J->fmt, get_code(J->q, bits, row_bytes, orow, oblk * 32 + i)) * s);
        if (J->hadamard) {
            or_fwht32(v);
            for (int i = 0; i < 32; i++) v[i] = v[i] * (1.0f / 32.0f);
        }
        if (J->ts)
            for (int i = 0; i < 32; i++) v[i] = v[i] * *J->ts;
        for (int i = 0; i < 32; i++) {
            const int64_t r = J->axis == OR_AXIS_ROW ? orow : oblk * 32 + i;
            const int64_t c = J->axis == OR_AXIS_ROW ? oblk * 32 + i : orow;
            J->out[r * J->cols + c] = v[i];
        }
    }
}

int or_dequantize(const uint8_t* q, const uint8_t* scales, const float* tensor_scale,
                  int fmt, int64_t rows, int64_t cols, int axis, int hadamard, float* out,
                  int nthreads)
{
    if (!shape_ok(rows, cols, cols, axis)) return -1;
    dq_job J = {q, scales, tensor_scale, fmt, rows, cols, axis, hadamard, out};
    parallel_for(rows * cols / 32, nthreads, dq_range, &J);
    return 0;
}

/* ------------------------------------------------------------------ */
/* GEMM ([MOSS, "GEMM Kernel 优化"]): the main loop works on the scaled    */
/* codes and the per-tensor scales are applied once at the end.  The     */
/* oracle writes out the definition: dequantize each operand exactly,    */
/* accumulate the dot products in double, multiply by alpha'.            */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint8_t* q; const uint8_t* s; int fmt; int64_t K;
    double dec[256];
} operand;

static void operand_init(operand* o, const uint8_t* q, const uint8_t* s, int fmt, int64_t K)
{
    o->q = q; o->s = s; o->fmt = fmt; o->K = K;
    for (unsigned c = 0; c < 256; c++) o->dec[c] = or_decode(fmt, c);
}

/* exact value of element (row, k) */
static double operand_at(const operand* o, int64_t row, int64_t k)
{
    const int bits = or_elem_bits(o->fmt);
    const unsigned code = get_code(o->q, bits, o->K * bits / 8, row, k);
    return o->dec[code] * or_decode_e8m0(o->s[row * (o->K / 32) + k / 32]);
}

static double alpha_prime(double alpha, const float* ta, const float* tb, int hadamard_k)
{
    double a = alpha;
    if (ta) a *= (double)*ta;
    if (tb) a *= (double)*tb;
    if (hadamard_k) a *= 1.0 / 32.0;
    return a;
}

typedef struct {
    operand A, B; int64_t M, N, K; double ap;
    double* Adq; double* Bdq;
    const int64_t* ii; const int64_t* jj;
    double* C; double* bound;
} gemm_job;

static void dq_rows_range(int64_t lo, int64_t hi, void* arg)
{
    /* rows [lo, hi) of the stacked (A; B) operands, dequantized exactly */
    gemm_job* J = (gemm_job*)arg;
    for (int64_t r = lo; r < hi; r++) {
        const operand* o = r < J->M ? &J->A : &J->B;
        double* dst = r < J->M ? &J->Adq[r * J->K] : &J->Bdq[(r - J->M) * J->K];
        const int64_t row = r < J->M ? r : r - J->M;
        for (int64_t k = 0; k < J->K; k++) dst[k] = operand_at(o, row, k);
    }
}

static void gemm_rows_range(int64_t lo, int64_t hi, void* arg)
{
    gemm_job* J = (gemm_job*)arg;
    for (int64_t i = lo; i < hi; i++)
        for (int64_t j = 0; j < J->N; j++) {
            const double* a = &J->Adq[i * J->K];
            const double* b = &J->Bdq[j * J->K];
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < J->K; k++) {
                acc += a[k] * b[k];
                mag += fabs(a[k]) * fabs(b[k]);
            }
            J->C[i * J->N + j] = J->ap * acc;
            if (J->bound) J->bound[i * J->N + j] = fabs(J->ap) * mag;
        }
}

static int gemm_args_ok(int fa, int fb, int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return 0;
    if (fa < 0 || fa > 2 || fb < 0 || fb > 2) return 0;
    return 1;
}

int or_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int fa,
            const uint8_t* qb, const uint8_t* sb, const float* tb, int fb,
            int64_t M, int64_t N, int64_t K, double alpha, int hadamard_k,
            double* C, double* bound, int nthreads)
{
    if (!gemm_args_ok(fa, fb, M, N, K)) return -1;
    gemm_job J;
    memset(&J, 0, sizeof J);
    operand_init(&J.A, qa, sa, fa, K);
    operand_init(&J.B, qb, sb, fb, K);
    J.M = M; J.N = N; J.K = K;
    J.ap = alpha_prime(alpha, ta, tb, hadamard_k);
    J.Adq = (double*)malloc(sizeof(double) * (size_t)(M * K));
    J.Bdq = (double*)malloc(sizeof(double) * (size_t)(N * K));
    if (!J.Adq || !J.Bdq) { free(J.Adq); free(J.Bdq); return -2; }
    J.C = C; J.bound = bound;
    parallel_for(M + N, nthreads, dq_rows_range, &J);
    parallel_for(M, nthreads, gemm_rows_range, &J);
    free(J.Adq);
    free(J.Bdq);
    return 0;
}

static void gemm_entries_range(int64_t lo, int64_t hi, void* arg)
{
    gemm_job* J = (gemm_job*)arg;
    for (int64_t t = lo; t < hi; t++) {
        const int64_t i = J->ii[t], j = J->jj[t];
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < J->K; k++) {
            const double a = operand_at(&J->A, i, k), b = operand_at(&J->B, j, k);
            acc += a * b;
            mag += fabs(a) * fabs(b);
        }
        J->C[t] = J->ap * acc;
        if (J->bound) J->bound[t] = fabs(J->ap) * mag;
    }
}

int or_gemm_entries(const uint8_t* qa, const uint8_t* sa, const float* ta, int fa,
                    const uint8_t* qb, const uint8_t* sb, const float* tb, int fb,
                    int64_t M, int64_t N, int64_t K, double alpha, int hadamard_k,
                    const int64_t* ii, const int64_t* jj, int64_t n,
                    double* C, double* bound, int nthreads)
{
    if (!gemm_args_ok(fa, fb, M, N, K)) return -1;
    for (int64_t t = 0; t < n; t++)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return -1;
    gemm_job J;
    memset(&J, 0, sizeof J);
    operand_init(&J.A, qa, sa, fa, K);
    operand_init(&J.B, qb, sb, fb, K);
    J.M = M; J.N = N; J.K = K;
    J.ap = alpha_prime(alpha, ta, tb, hadamard_k);
    J.ii = ii; J.jj = jj; J.C = C; J.bound = bound;
    parallel_for(n, nthreads, gemm_entries_range, &J);
    return 0;
}

/* ------------------------------------------------------------------ */
/* FP8 optimizer states with dynamic range expansion ([COAT, "解決方案：  */
/* 動態範圍擴充套件"]).  The page states the goal -- an expansion function */
/* applied before quantization, with one parameter k per quantization  */
/* group computed on the fly, that stretches the group's max/min ratio */
/* to the FP8 format's (about 2e5 for E4M3) -- but its formula did not */
/* survive.  Reading, after the COAT paper the page cites: f(x) =      */
/* sign(x)|x|^k.  Per group, with the magnitudes normalised by the     */
/* group's largest one so that every power stays in fp32 range:        */
/*   u = |x| / amax,  k = log2(R_fmt) / log2(amax / amin_nonzero),     */
/*   y = sign(x) * u^k * Fmax  -> FP8 code (RNE, saturating),          */
/* so the largest magnitude maps to Fmax and the smallest nonzero one  */
/* to Fmax / R_fmt = the smallest subnormal; R_fmt = Fmax / (smallest  */
/* subnormal).  Stored per group: amax and k.  Inverse:                */
/*   x = sign(q) * amax * (|decode(q)| / Fmax)^(1/k).                  */
/* The powers go through log2 and exp2.  So that the codes are a plain */
/* function of fp32 arithmetic, both are written out as fixed fp32     */
/* polynomial evaluations, each step a single IEEE operation (a fused  */
/* multiply-add where written, `fmaf`), in the order written.          */
/* log2: x = m * 2^e with m in (sqrt(1/2), sqrt(2)), z = m - 1 (exact),*/
/* log2(x) = e + z * P(z), P of degree 8 fitted to log2(1+z)/z on that */
/* range (least squares on Chebyshev nodes, coefficients rounded to    */
/* fp32; about 2 ulp).  exp2: y = n + z with n = floor(y + 1/2),       */
/* z = y - n (exact), 2^z from a degree-6 fit on [-1/2, 1/2] with a     */
/* constant term of exactly 1 (about 1.3 ulp), then 2^n by ldexp.      */
/* ------------------------------------------------------------------ */
float or_log2_fp32(float x)
{
    /* x > 0 (finite or +Inf) */
    int e = 0;
    if (x < 0x1p-126f) { x = x * 0x1p32f; e = -32; }          /* subnormal: exact scaling */
    uint32_t b;
    memcpy(&b, &x, 4);
    e += (int)((b >> 23) & 0xFFu) - 127;
    b = (b & 0x7FFFFFu) | 0x3F800000u;
    float m;
    memcpy(&m, &b, 4);
    if (m > 1.41421356f) { m = m * 0.5f; e += 1; }
    const float z = m - 1.0f;                                  /* exact (Sterbenz) */
    float p = 0x1.025a88p-3f;
    p = fmaf(p, z, -0x1.a8cd06p-3f);
    p = fmaf(p, z, 0x1.b9b144p-3f);
    p = fmaf(p, z, -0x1.e94efep-3f);
    p = fmaf(p, z, 0x1.26d40cp-2f);
    p = fmaf(p, z, -0x1.715c9cp-2f);
    p = fmaf(p, z, 0x1.ec73d4p-2f);
    p = fmaf(p, z, -0x1.71547p-1f);
    p = fmaf(p, z, 0x1.715476p+0f);
    return fmaf(z, p, (float)e);
}

float or_exp2_fp32(float y)
{
    if (y != y) return y;
    if (y >= 128.0f) return INFINITY;
    if (y < -150.0f) return 0.0f;
    const float n = floorf(y + 0.5f);
    const float z = y - n;                                     /* exact, |z| <= 1/2 */
    float p = 0x1.41a7p-13f;
    p = fmaf(p, z, 0x1.5f44f4p-10f);
    p = fmaf(p, z, 0x1.3b2dfep-7f);
    p = fmaf(p, z, 0x1.c6aed6p-5f);
    p = fmaf(p, z, 0x1.ebfbdap-3f);
    p = fmaf(p, z, 0x1.62e43p-1f);
    p = fmaf(p, z, 1.0f);
    return ldexpf(p, (int)n);
}

/* u^k for u >= 0 */
float or_pow_fp32(float u, float k)
{
    if (u == 0.0f) return 0.0f;
    return or_exp2_fp32(k * or_log2_fp32(u));
}

/* log2 of the format's dynamic range Fmax / smallest subnormal, as an fp32
 * constant: E4M3 448 / 2^-9, E5M2 57344 / 2^-16 */
static float log2_range(int fmt)
{
    return fmt == OR_E4M3 ? 17.8073549f : 31.8073549f;
}

typedef struct {
    const float* x; int64_t group; int fmt;
    uint8_t* q; float* amax; float* kexp;
} os_job;

static void os_quant_range(int64_t lo, int64_t hi, void* arg)
{
    const os_job* J = (const os_job*)arg;
    const int64_t G = J->group;
    const float fmax = (float)or_fmax(J->fmt);
    for (int64_t g = lo; g < hi; g++) {
        const float* x = J->x + g * G;
        uint8_t* q = J->q + g * G;
        int finite = 1;
        float amax = 0.0f, amin = INFINITY;
        for (int64_t i = 0; i < G; i++) {
            const float a = fabsf(x[i]);
            if (!isfinite(a)) finite = 0;
            if (a > amax) amax = a;
            if (a > 0.0f && a < amin) amin = a;
        }
        if (!finite) {
            for (int64_t i = 0; i < G; i++) q[i] = 0x7F;
            J->amax[g] = NAN;
            J->kexp[g] = NAN;
            continue;
        }
        if (amax == 0.0f) {                          /* all zero: signed zeros, unit parameters */
            for (int64_t i = 0; i < G; i++) q[i] = signbit(x[i]) ? (uint8_t)0x80 : (uint8_t)0x00;
            J->amax[g] = 1.0f;
            J->kexp[g] = 1.0f;
            continue;
        }
        const float r = amax / amin;
        const float k = r > 1.0f ? log2_range(J->fmt) / or_log2_fp32(r) : 1.0f;
        for (int64_t i = 0; i < G; i++) {
            const float u = fabsf(x[i]) / amax;
            float y = or_pow_fp32(u, k) * fmax;
            if (signbit(x[i])) y = -y;
            q[i] = (uint8_t)or_encode_rne(J->fmt, (double)y);
        }
        J->amax[g] = amax;
        J->kexp[g] = k;
    }
}

int or_optstate_quantize(const float* x, int64_t n, int64_t group, int fmt, uint8_t* q, float* amax,
                         float* kexp, int nthreads)
{
    if (group <= 0 || n <= 0 || n % group != 0 || (fmt != OR_E4M3 && fmt != OR_E5M2)) return -1;
    os_job J = {x, group, fmt, q, amax, kexp};
    parallel_for(n / group, nthreads, os_quant_range, &J);
    return 0;
}

static void os_dequant_range(int64_t lo, int64_t hi, void* arg)
{
    const os_job* J = (const os_job*)arg;              /* x is the output here */
    const int64_t G = J->group;
    const float fmax = (float)or_fmax(J->fmt);
    float* out = (float*)J->x;
    for (int64_t g = lo; g < hi; g++) {
        const float amax = J->amax[g], k = J->kexp[g];
        const float kinv = 1.0f / k;
        for (int64_t i = 0; i < G; i++) {
            const unsigned c = J->q[g * G + i];
            const float v = (float)or_decode(J->fmt, c);
            float a = amax * or_pow_fp32(fabsf(v) / fmax, kinv);
            if (v != v || amax != amax || k != k) a = NAN;
            out[g * G + i] = (c & 0x80u) ? -a : a;
        }
    }
}

int or_optstate_dequantize(const uint8_t* q, const float* amax, const float* kexp, int64_t n, int64_t group,
                           int fmt, float* out, int nthreads)
{
    if (group <= 0 || n <= 0 || n % group != 0 || (fmt != OR_E4M3 && fmt != OR_E5M2)) return -1;
    os_job J = {out, group, fmt, (uint8_t*)q, (float*)amax, (float*)kexp};
    parallel_for(n / group, nthreads, os_dequant_range, &J);
    return 0;
}

/* ------------------------------------------------------------------ */
/* nvfp routes ([FAF, "格式感知融合的设计思路"]: native mxfp, global nvfp  */
/* and CTA-local nvfp, each quantization producer bound to its scale  */
/* domain and consumer layout; [FAF, "FP4加速为何常常纸上富贵"]: nvfp is  */
/* block scaling, one scale per block of values).  The pages fix       */
/* neither block size nor scale format; reading: NVIDIA's published    */
/* NVFP4 -- E2M1 elements in blocks of 16 along the stored row, an     */
/* unsigned E4M3 scale per block, and an FP32 second-level scale       */
/* s = amax / (6 * 448) so that every block scale fits E4M3:           */
/*   global: one s over the tensor;                                    */
/*   local:  one s per panel of 32 stored rows (the rows one GEMM tile  */
/*           consumes over all of K), no reduction across panels.      */
/* Per block: den = RN(6 s); sb = E4M3_RNE_sat(RN(amax_b / den));       */
/* d = RN(decode(sb) * s); r = RN(1 / d); code_i = E2M1_RNE_sat(RN(v_i * */
/* r)).  A zero block scale gives signed zeros; a block holding a NaN  */
/* or Inf gets scale code 0x7F (E4M3 NaN) and zero codes.              */
/* ------------------------------------------------------------------ */
#define NV_PANEL 32

typedef struct {
    const void* x; int src; int64_t rows, cols, ld; int axis, local;
    uint8_t* q; uint8_t* s16; const float* ts;
} nv_job;

/* element (stored row sr, position c along it) of the source */
static float nv_src(const nv_job* J, int64_t sr, int64_t c)
{
    return J->axis == OR_AXIS_ROW ? load_src(J->x, J->src, sr * J->ld + c)
                                  : load_src(J->x, J->src, c * J->ld + sr);
}

static void nv_quant_range(int64_t lo, int64_t hi, void* arg)
{
    const nv_job* J = (const nv_job*)arg;
    const int64_t L = J->axis == OR_AXIS_ROW ? J->cols : J->rows;       /* stored row length */
    const int64_t nb = L / 16;
    for (int64_t sr = lo; sr < hi; sr++) {
        const float s = J->ts[J->local ? sr / NV_PANEL : 0];
        for (int64_t b = 0; b < nb; b++) {
            float v[16];
            float amax = 0.0f;
            int finite = 1;
            for (int i = 0; i < 16; i++) {
                v[i] = nv_src(J, sr, b * 16 + i);
                if (!isfinite(v[i])) finite = 0;
                if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            unsigned sb;
            unsigned codes[16];
            if (!finite || s != s) {
                sb = 0x7F;
                for (int i = 0; i < 16; i++) codes[i] = 0;
            } else {
                const float den = 6.0f * s;
                sb = or_encode_rne(OR_E4M3, (double)(amax / den)) & 0x7Fu;   /* unsigned scale */
                const float ds = (float)or_decode(OR_E4M3, sb);
                if (ds == 0.0f) {
                    for (int i = 0; i < 16; i++) codes[i] = signbit(v[i]) ? 0x8u : 0x0u;
                } else {
                    const float d = ds * s;
                    const float r = 1.0f / d;
                    for (int i = 0; i < 16; i++) codes[i] = or_encode_rne(OR_E2M1, (double)(v[i] * r));
                }
            }
            J->s16[sr * nb + b] = (uint8_t)sb;
            for (int i = 0; i < 16; i++) put_code(J->q, 4, L / 2, sr, b * 16 + i, codes[i]);
        }
    }
}

/* second-level scale of one domain: amax / (6 * 448), 1 for an all-zero
 * domain, NaN when it holds a NaN or Inf */
static float nv_domain_scale(const nv_job* J, int64_t sr0, int64_t sr1)
{
    const int64_t L = J->axis == OR_AXIS_ROW ? J->cols : J->rows;
    float amax = 0.0f;
    for (int64_t sr = sr0; sr < sr1; sr++)
        for (int64_t c = 0; c < L; c++) {
            const float a = fabsf(nv_src(J, sr, c));
            if (!isfinite(a)) return NAN;
            if (a > amax) amax = a;
        }
    return amax == 0.0f ? 1.0f : amax / 2688.0f;
}

int or_nvfp_quantize(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int axis, int local,
                     uint8_t* q, uint8_t* s16, float* tscale, int nthreads)
{
    const int64_t SR = axis == OR_AXIS_ROW ? rows : cols, L = axis == OR_AXIS_ROW ? cols : rows;
    if (rows <= 0 || cols <= 0 || ld < cols || L % 16 != 0) return -1;
    nv_job J = {x, src, rows, cols, ld, axis, local, q, s16, tscale};
    if (local) {
        for (int64_t p = 0; p * NV_PANEL < SR; p++)
            tscale[p] = nv_domain_scale(&J, p * NV_PANEL, (p + 1) * NV_PANEL < SR ? (p + 1) * NV_PANEL : SR);
    } else {
        tscale[0] = nv_domain_scale(&J, 0, SR);
    }
    parallel_for(SR, nthreads, nv_quant_range, &J);
    return 0;
}

/* x_hat = RN(RN(decode(code) * decode(sb)) * s): the first product is exact
 * (at most 6 significant bits), the second rounds once */
int or_nvfp_dequantize(const uint8_t* q, const uint8_t* s16, const float* tscale, int64_t rows, int64_t cols,
                       int axis, int local, float* out)
{
    const int64_t SR = axis == OR_AXIS_ROW ? rows : cols, L = axis == OR_AXIS_ROW ? cols : rows;
    if (rows <= 0 || cols <= 0 || L % 16 != 0) return -1;
    for (int64_t sr = 0; sr < SR; sr++) {
        const float s = tscale[local ? sr / NV_PANEL : 0];
        for (int64_t c = 0; c < L; c++) {
            const float ds = (float)or_decode(OR_E4M3, s16[sr * (L / 16) + c / 16]);
            const float e = (float)or_decode(OR_E2M1, get_code(q, 4, L / 2, sr, c));
            const float v = (e * ds) * s;
            if (axis == OR_AXIS_ROW) out[sr * cols + c] = v;
            else out[c * cols + sr] = v;
        }
    }
    return 0;
}

typedef struct {
    const uint8_t *qa, *sa, *qb, *sb; const float *ta, *tb; int la, lb;
    int64_t N, K; double alpha; double *C, *bound;
} nvg_job;

static double nv_elem(const uint8_t* q, const uint8_t* s, int64_t K, int64_t row, int64_t k)
{
    return or_decode(OR_E2M1, get_code(q, 4, K / 2, row, k)) * or_decode(OR_E4M3, s[row * (K / 16) + k / 16]);
}

/* one output entry and its bound */
static void nvg_entry(const nvg_job* J, int64_t i, int64_t j, double* c, double* bound)
{
    const double sA = J->ta[J->la ? i / NV_PANEL : 0];
    const double sB = J->tb[J->lb ? j / NV_PANEL : 0];
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < J->K; k++) {
        const double a = nv_elem(J->qa, J->sa, J->K, i, k), b = nv_elem(J->qb, J->sb, J->K, j, k);
        acc += a * b;
        mag += fabs(a * b);
    }
    const double ap = J->alpha * sA * sB;
    *c = ap * acc;
    *bound = fabs(ap) * mag;
}

static void nvg_range(int64_t lo, int64_t hi, void* arg)
{
    const nvg_job* J = (const nvg_job*)arg;
    for (int64_t i = lo; i < hi; i++)
        for (int64_t j = 0; j < J->N; j++)
            nvg_entry(J, i, j, &J->C[i * J->N + j], &J->bound[i * J->N + j]);
}

typedef struct {
    nvg_job g; const int64_t *ii, *jj;
} nvg_entries_job;

static void nvg_entries_range(int64_t lo, int64_t hi, void* arg)
{
    const nvg_entries_job* E = (const nvg_entries_job*)arg;
    for (int64_t e = lo; e < hi; e++) nvg_entry(&E->g, E->ii[e], E->jj[e], &E->g.C[e], &E->g.bound[e]);
}

/* C[i][j] = alpha * sA(i) * sB(j) * sum_k Ahat[i][k] Bhat[j][k] in double, with
 * Ahat = decode(code) * decode(block scale) (exact) and sA(i) the second-level
 * scale of row i's domain (one, or one per 32-row panel); bound as or_gemm. */
int or_nvfp_gemm(const uint8_t* qa, const uint8_t* sa, const float* ta, int local_a,
                 const uint8_t* qb, const uint8_t* sb, const float* tb, int local_b,
                 int64_t M, int64_t N, int64_t K, double alpha, double* C, double* bound, int nthreads)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return -1;
    nvg_job J = {qa, sa, qb, sb, ta, tb, local_a, local_b, N, K, alpha, C, bound};
    parallel_for(M, nthreads, nvg_range, &J);
    return 0;
}

/* the entries (ii[e], jj[e]) of or_nvfp_gemm's C and bound */
int or_nvfp_gemm_entries(const uint8_t* qa, const uint8_t* sa, const float* ta, int local_a,
                         const uint8_t* qb, const uint8_t* sb, const float* tb, int local_b,
                         int64_t M, int64_t N, int64_t K, double alpha, const int64_t* ii, const int64_t* jj,
                         int64_t n, double* C, double* bound, int nthreads)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0 || n < 0) return -1;
    for (int64_t e = 0; e < n; e++)
        if (ii[e] < 0 || ii[e] >= M || jj[e] < 0 || jj[e] >= N) return -1;
    nvg_entries_job E = {{qa, sa, qb, sb, ta, tb, local_a, local_b, N, K, alpha, C, bound}, ii, jj};
    parallel_for(n, nthreads, nvg_entries_range, &E);
    return 0;
}
