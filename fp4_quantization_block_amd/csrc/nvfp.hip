// nvfp.hip -- the nvfp routes: NVFP4 quantization with a global or a
// CTA-local second-level scale, its dequantization, and the GEMM that
// consumes it on gfx950.
//
// [FAF, "格式感知融合的设计思路"]: the method binds every quantization
// producer to its scale domain and its consumer's layout, for native mxfp,
// global nvfp and CTA-local nvfp; [FAF, "FP4加速为何常常纸上富贵"]: nvfp is
// block scaling, one scale per block.  The pages fix neither block size nor
// scale format; the reading is NVIDIA's NVFP4: E2M1 elements in blocks of
// 16 along the stored row, an unsigned E4M3 scale per block, and an FP32
// second-level scale s = amax / (6 * 448) that keeps every block scale
// inside E4M3:
//   global: one s over the tensor (a reduction over all of it first);
//   local:  one s per panel of 32 stored rows -- the rows one GEMM tile
//           consumes over all of K -- so each producer workgroup scales its
//           own panel with no reduction across workgroups, and the GEMM
//           applies the panel scales in its epilogue.
// Per block (the arithmetic of the oracle, each step rounded once):
//   den = 6 * s;  sb = E4M3_RNE_sat(amax_b / den);  d = decode(sb) * s;
//   r = 1 / d;    code_i = E2M1_RNE_sat(v_i * r)
// with signed zeros for a zero block scale, and scale code 0x7F (E4M3 NaN)
// with zero codes for a block holding a NaN or Inf.  Copies are stored like
// the mx copies: row copy [rows][cols/2] bytes, column copy transposed
// [cols][rows/2], two codes per byte (element 2j in the low nibble), block
// scales [stored rows][row length / 16].
//
// The consumer.  gfx950's block-scaled matrix instruction takes one E8M0
// (power-of-two) scale per 32 elements; an E4M3 scale per 16 is not a
// power of two, so nvfp operands cannot ride on it.  The GEMM dequantizes in
// its main loop instead, exactly: an E4M3 scale is f * 2^E with f an integer
// <= 15, the FP4 -> f16 converter applies 2^E, a packed f16 multiply by f
// is exact (E2M1 times f needs at most 6 significant bits), and the f16
// matrix instruction multiplies exactly and accumulates in fp32.  This is
// the main-loop dequantization that [MOSS, "GEMM Kernel 优化"] shows eating
// the gain -- the price of this scale domain on this hardware: the f16
// matrix peak is a quarter of the FP4 one.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int NV_PANEL = 32;                       // stored rows per local scale domain

template <int SRC> __device__ __forceinline__ float src_at(const void* x, int64_t i)
{
    if constexpr (SRC == SRC_BF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[i] << 16);
    else return ((const float*)x)[i];
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// exact fp32 value of an E4M3 code
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 15 && m == 7) v = __builtin_nanf("");
    else if (e == 0) v = (float)m * exp2i(-9);
    else v = (float)(8u | m) * exp2i((int)e - 10);
    return (c & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------------------
// second-level scales
// ---------------------------------------------------------------------------
// amax key (|x| bits; NaN above Inf above finite) of stored rows
// [32 p, 32 p + 32) of the copy, one workgroup per panel p
template <int SRC, bool ROW>
__global__ __launch_bounds__(256) void k_nv_panel_amax(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                                       int64_t npanels, int local, float* ts, uint32_t* keys)
{
    const int64_t SR = ROW ? rows : cols, L = ROW ? cols : rows;
    for (int64_t p = blockIdx.x; p < npanels; p += gridDim.x) {
        const int64_t r0 = p * NV_PANEL, r1 = min(r0 + NV_PANEL, SR);
        uint32_t key = 0;
        if (ROW) {                                   // panel rows are source rows: walk each along its length
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = threadIdx.x; c < L; c += 256)
                    key = max(key, __float_as_uint(src_at<SRC>(x, r * ld + c)) & 0x7FFFFFFFu);
        } else {                                     // panel rows are source columns: 32 per source row
            for (int64_t i = threadIdx.x; i < (r1 - r0) * L; i += 256) {
                const int64_t r = i / (r1 - r0), c = r0 + i % (r1 - r0);
                key = max(key, __float_as_uint(src_at<SRC>(x, r * ld + c)) & 0x7FFFFFFFu);
            }
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
        __shared__ uint32_t red[4];
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
        __syncthreads();
        if (threadIdx.x == 0) {
            key = max(max(red[0], red[1]), max(red[2], red[3]));
            if (local) {
                ts[p] = key >= 0x7F800000u ? __builtin_nanf("") : key == 0 ? 1.0f : __uint_as_float(key) / 2688.0f;
            } else {
                keys[p] = key;
            }
        }
        __syncthreads();
    }
}

// global: one workgroup reduces the panel keys into the tensor's scale
__global__ __launch_bounds__(256) void k_nv_global_scale(const uint32_t* keys, int64_t n, float* ts)
{
    uint32_t key = 0;
    for (int64_t i = threadIdx.x; i < n; i += 256) key = max(key, keys[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        key = max(max(red[0], red[1]), max(red[2], red[3]));
        ts[0] = key >= 0x7F800000u ? __builtin_nanf("") : key == 0 ? 1.0f : __uint_as_float(key) / 2688.0f;
    }
}

// ---------------------------------------------------------------------------
// quantize: one thread per block of 16 along the stored row
// ---------------------------------------------------------------------------
template <int SRC, bool ROW>
__global__ __launch_bounds__(256) void k_nv_quant(const void* x, int64_t rows, int64_t cols, int64_t ld, int local,
                                                  const float* ts, uint8_t* q, uint8_t* s16)
{
    const int64_t SR = ROW ? rows : cols, L = ROW ? cols : rows, nb = L / 16, total = SR * nb;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        // row copy: consecutive threads walk a stored row's blocks; column copy:
        // consecutive threads take neighbouring source columns (coalesced reads)
        const int64_t sr = ROW ? t / nb : t % SR, b = ROW ? t % nb : t / SR;
        const float s = ts[local ? sr / NV_PANEL : 0];
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; i++)
            v[i] = ROW ? src_at<SRC>(x, sr * ld + b * 16 + i) : src_at<SRC>(x, (b * 16 + i) * ld + sr);
        uint32_t key = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) key = max(key, __float_as_uint(v[i]) & 0x7FFFFFFFu);
        uint32_t sb;
        uint32_t w0 = 0, w1 = 0;                     // 16 codes
        if (key >= 0x7F800000u || s != s) {
            sb = 0x7Fu;
        } else {
            const float den = 6.0f * s;
            const float bv = __uint_as_float(key) / den;
            sb = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fmax<E4M3>(bv), 0.0f, 0, false) & 0x7Fu;
            const float ds = e4m3_value(sb);
            if (ds == 0.0f) {
#pragma unroll
                for (int i = 0; i < 8; i++) w0 |= (__float_as_uint(v[i]) >> 31) << (4 * i + 3);
#pragma unroll
                for (int i = 0; i < 8; i++) w1 |= (__float_as_uint(v[8 + i]) >> 31) << (4 * i + 3);
            } else {
                const float d = ds * s;
                const float r = 1.0f / d;
                float y[16];
#pragma unroll
                for (int i = 0; i < 16; i++) y[i] = clamp_fmax<E2M1>(v[i] * r);
                w0 = cvt8_fp4(y);
                w1 = cvt8_fp4(y + 8);
            }
        }
        s16[sr * nb + b] = (uint8_t)sb;
        *(uint2*)(q + sr * (L / 2) + b * 8) = make_uint2(w0, w1);
    }
}

// dequantize: one thread per block; x_hat = (code * decode(sb)) * s, the
// first product exact
template <bool ROW, int OUTT>
__global__ __launch_bounds__(256) void k_nv_dequant(const uint8_t* q, const uint8_t* s16, const float* ts,
                                                    int64_t rows, int64_t cols, int local, void* out)
{
    const int64_t SR = ROW ? rows : cols, L = ROW ? cols : rows, nb = L / 16, total = SR * nb;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t sr = ROW ? t / nb : t % SR, b = ROW ? t % nb : t / SR;
        const float s = ts[local ? sr / NV_PANEL : 0];
        const float ds = e4m3_value(s16[sr * nb + b]);
        const uint2 w = *(const uint2*)(q + sr * (L / 2) + b * 8);
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t c = ((i < 8 ? w.x : w.y) >> (4 * (i & 7))) & 0xFu;
            // E2M1 magnitude: exponent field m >> 1, mantissa bit m & 1
            const uint32_t m = c & 7u, ef = m >> 1;
            const float half = 0.5f * (float)(m & 1u);
            const float mag = ef == 0 ? half : (1.0f + half) * exp2i((int)ef - 1);
            const float ev = (c & 8u) ? -mag : mag;
            const float val = (ev * ds) * s;
            const int64_t idx = ROW ? sr * cols + b * 16 + i : (b * 16 + i) * cols + sr;
            if constexpr (OUTT == 0) ((float*)out)[idx] = val;
            else ((uint16_t*)out)[idx] = bf16_rne(val);
        }
    }
}

// ---------------------------------------------------------------------------
// k_nv_gemm: C = alpha * sA(i) * sB(j) * sum_k Ahat[i][k] Bhat[j][k] on nvfp
// operands (A [M][K] and B [N][K] row copies as the quantizer writes them;
// sA(i), sB(j) the second-level scale of the row's domain).  256x256 tile
// per 256-thread workgroup, one wave per SIMD computing a 128x128 quarter
// (4x4 f16 MFMA 32x32x16 tiles, all 256 accumulators); K advances 64
// elements per stage.  Each stage's codes and block scales are loaded into
// registers a stage ahead, dequantized exactly to f16 (converter with 2^E,
// packed multiply by the integer factor), and written to the other of two
// LDS stage buffers (rows of 128 bytes whose 16-byte chunks are
// XOR-swizzled by (row >> 1) & 7, conflict-free for the fragment reads).
// The second-level scales are applied once per output in the epilogue.
// ---------------------------------------------------------------------------
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16acc __attribute__((ext_vector_type(16)));

constexpr int NBM = 256, NBK = 64, NROWB = NBK * 2;   // tile rows, K per stage, f16 bytes per tile row

__device__ __forceinline__ int nv_swz(int row, int chunk) { return row * NROWB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// one 16-byte chunk of codes (32 elements, two blocks) and its two block
// scales -> 32 exact f16 values into LDS row `row`, chunks 4*half .. 4*half+3
__device__ __forceinline__ void nv_dequant_chunk(uint8_t* tile, int row, int half, uint4 codes, uint32_t sc2)
{
    float p2[2];
    _Float16 fct[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const uint32_t sb = (sc2 >> (8 * b)) & 0xFFu, e = (sb >> 3) & 15u, m = sb & 7u;
        // E4M3 scale = f * 2^E: subnormal f = m, E = -9; normal f = 8 + m, E = e - 10
        p2[b] = exp2i(e == 0 ? -9 : (int)e - 10);
        fct[b] = sb == 0x7Fu ? (_Float16)__builtin_nanf("") : (_Float16)(float)(e == 0 ? m : 8u + m);
    }
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {                    // 16-byte output chunk q: code bytes 4q .. 4q+3
        const int b = q / 2;                         // bytes 0-7: block 0, bytes 8-15: block 1
        const h2 f2 = {fct[b], fct[b]};
        h2 v[4];
        v[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], p2[b], 0) * f2;
        v[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], p2[b], 1) * f2;
        v[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], p2[b], 2) * f2;
        v[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], p2[b], 3) * f2;
        const h8 out = {v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
        *(h8*)(tile + nv_swz(row, 4 * half + q)) = out;
    }
}

template <int OUTT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_nv_gemm(NvGemmJob g, int tiles_m, int tiles_n)
{
    __shared__ __align__(16) uint8_t lA[2][NBM * NROWB];
    __shared__ __align__(16) uint8_t lB[2][NBM * NROWB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;

    // tile order: workgroups dealt round-robin to the 8 XCDs; each XCD takes a
    // contiguous range of tiles in row-major order of 4-row groups
    int t = blockIdx.x;
    const int total = tiles_m * tiles_n;
    if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
    const int grp = 4 * tiles_n, first = (t / grp) * 4, nrows = min(4, tiles_m - first);
    const int tm = first + (t % grp) % nrows, tn = (t % grp) / nrows;
    const int64_t m0 = (int64_t)tm * NBM, n0 = (int64_t)tn * NBM;
    const int64_t kcb = g.K / 2, ksb = g.K / 16;
    const int nst = (int)(g.K / NBK);

    auto rsrc = [&](const uint8_t* base, int64_t first_row, int64_t rows, int64_t row_bytes) __attribute__((always_inline)) {
        int64_t n = (rows - first_row) * row_bytes;
        n = n < 0 ? 0 : n > 0xFFFFFFFFll ? 0xFFFFFFFFll : n;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + first_row * row_bytes), (short)0, (int)(uint32_t)n,
                                                 0x00020000);
    };
    const auto rA = rsrc(g.qa, m0, g.M, kcb), rB = rsrc(g.qb, n0, g.N, kcb);
    const auto rSA = rsrc(g.sa, m0, g.M, ksb), rSB = rsrc(g.sb, n0, g.N, ksb);

    // loads of a stage: chunk c = tid + 256 p (p = 0, 1) is row c / 2, half c % 2
    uint4 cA[2], cB[2];
    uint32_t sA[2], sB[2];
    auto gload = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int c = tid + 256 * p, row = c >> 1, half = c & 1;
            const uint32_t co = (uint32_t)(row * kcb) + (uint32_t)(half * 16);
            const uint32_t so = (uint32_t)(row * ksb) + (uint32_t)(half * 2);
            cA[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rA, co, s * 32, 0));
            cB[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rB, co, s * 32, 0));
            sA[p] = __builtin_amdgcn_raw_buffer_load_b16(rSA, so, s * 4, 0);
            sB[p] = __builtin_amdgcn_raw_buffer_load_b16(rSB, so, s * 4, 0);
        }
    };
    auto dq_write = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const int c = tid + 256 * p, row = c >> 1, half = c & 1;
            nv_dequant_chunk(lA[buf], row, half, cA[p], sA[p]);
            nv_dequant_chunk(lB[buf], row, half, cB[p], sB[p]);
        }
    };

    f16acc acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    gload(0);
    dq_write(0);
    if (nst > 1) gload(1);
    __syncthreads();
    for (int s = 0; s < nst; s++) {
        const int cur = s & 1;
#pragma unroll
        for (int ks = 0; ks < NBK / 16; ks++) {
            h8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = *(const h8*)(lA[cur] + nv_swz(wm * 128 + i * 32 + l32, 2 * ks + h));
                b[i] = *(const h8*)(lB[cur] + nv_swz(wn * 128 + i * 32 + l32, 2 * ks + h));
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < nst) {
            dq_write(cur ^ 1);                       // stage s+1 into the buffer stage s-1 used
            if (s + 2 < nst) gload(s + 2);
        }
        __syncthreads();
    }

    // epilogue: alpha and the two second-level scales once per output
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t col = n0 + wn * 128 + j * 32 + l32;
            if (col >= g.N) continue;
            const float sbv = g.tb[g.lb ? col / NV_PANEL : 0];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                if (row >= g.M) continue;
                const float sav = g.ta[g.la ? row / NV_PANEL : 0];
                const float ap = (g.alpha * sav) * sbv;
                const float v = acc[i][j][r] * ap;
                if constexpr (OUTT == 0) ((float*)g.c)[row * g.ldc + col] = v;
                else ((uint16_t*)g.c)[row * g.ldc + col] = bf16_rne(v);
            }
        }
}

// enough workgroups to cover the blocks, at most 16 per CU (grid-stride loops)
unsigned nv_grid(int64_t items)
{
    int64_t wg = (items + 255) / 256;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t cap = (int64_t)cus * 16;
    return (unsigned)(wg < 1 ? 1 : (wg < cap ? wg : cap));
}

template <int SRC, bool ROW>
hipError_t launch_nv_quant(const NvQuantJob& j, hipStream_t st)
{
    const int64_t SR = ROW ? j.rows : j.cols, L = ROW ? j.cols : j.rows;
    const int64_t npanels = (SR + NV_PANEL - 1) / NV_PANEL;
    const unsigned pg = (unsigned)(npanels < 4096 ? npanels : 4096);
    // global: per-panel keys parked in the code array, which the quantize
    // kernel overwrites afterwards (SR * L / 2 >= 8 * SR >= 4 * npanels bytes)
    k_nv_panel_amax<SRC, ROW><<<pg, 256, 0, st>>>(j.x, j.rows, j.cols, j.ld, npanels, j.local, j.ts,
                                                   (uint32_t*)j.q);
    if (!j.local) k_nv_global_scale<<<1, 256, 0, st>>>((const uint32_t*)j.q, npanels, j.ts);
    k_nv_quant<SRC, ROW><<<nv_grid(SR * (L / 16)), 256, 0, st>>>(j.x, j.rows, j.cols, j.ld, j.local, j.ts, j.q, j.s16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nv_quantize(const NvQuantJob& j, hipStream_t stream)
{
    const bool row = j.axis == 0;
    if (j.src == SRC_BF16) return row ? launch_nv_quant<SRC_BF16, true>(j, stream) : launch_nv_quant<SRC_BF16, false>(j, stream);
    return row ? launch_nv_quant<SRC_F32, true>(j, stream) : launch_nv_quant<SRC_F32, false>(j, stream);
}

hipError_t launch_nv_dequantize(const NvQuantJob& j, const void* out, int out_dtype, hipStream_t stream)
{
    const int64_t SR = j.axis == 0 ? j.rows : j.cols, L = j.axis == 0 ? j.cols : j.rows;
    const unsigned grid = nv_grid(SR * (L / 16));
    void* o = const_cast<void*>(out);
    if (j.axis == 0) {
        if (out_dtype == 0) k_nv_dequant<true, 0><<<grid, 256, 0, stream>>>(j.q, j.s16, j.ts, j.rows, j.cols, j.local, o);
        else k_nv_dequant<true, 1><<<grid, 256, 0, stream>>>(j.q, j.s16, j.ts, j.rows, j.cols, j.local, o);
    } else {
        if (out_dtype == 0) k_nv_dequant<false, 0><<<grid, 256, 0, stream>>>(j.q, j.s16, j.ts, j.rows, j.cols, j.local, o);
        else k_nv_dequant<false, 1><<<grid, 256, 0, stream>>>(j.q, j.s16, j.ts, j.rows, j.cols, j.local, o);
    }
    return hipGetLastError();
}

hipError_t launch_nv_gemm(const NvGemmJob& j, hipStream_t stream)
{
    const int tiles_m = (int)((j.M + NBM - 1) / NBM), tiles_n = (int)((j.N + NBM - 1) / NBM);
    const unsigned grid = (unsigned)(tiles_m * tiles_n);
    if (j.out_dtype == 0) k_nv_gemm<0><<<grid, 256, 0, stream>>>(j, tiles_m, tiles_n);
    else k_nv_gemm<1><<<grid, 256, 0, stream>>>(j, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace mx
