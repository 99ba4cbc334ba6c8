// quant.hip -- MX quantization kernels for gfx950.
//
// Method ([MOSS, "两级缩放实现"], [FAF, "两个关键的数值技巧"], OCP MX v1.0):
// per 32-element block along the block axis: optional two-level division by
// the FP32 tensor scale, optional fixed-sign 32-point Hadamard, block amax ->
// E8M0 shared exponent, exact power-of-two scaling, saturating RNE or
// Philox-driven stochastic rounding, packing.  The dual-layout form writes the
// row copy and the transposed column copy from one read of the source
// ([FAF, "格式感知融合的设计思路"]: producer and consumer layout designed
// together).
//
// Sources:
//   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
//   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践"
//
// Work decomposition of the general kernel: a 256-thread workgroup is four
// waves stacked along the rows; each wave owns a 32-row strip and each lane a
// 32-row x 4-column sub-tile held in registers.  Column blocks (32x1) are
// then entirely inside one lane; row blocks (1x32) span 8 adjacent lanes and
// are reduced with cross-lane shuffles.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int kSubW = 4;          // columns per lane
constexpr int kWaves = 4;         // waves per workgroup (stacked along rows)

struct QArgs {
    const void* x;
    int64_t rows, cols, ld;
    uint8_t* q_row; uint8_t* s_row;
    uint8_t* q_col; uint8_t* s_col;
    const float* tscale;
    uint32_t k0, k1, offset;
    int sr, hadamard, two_level;
};

// FP32 tensor scale s_t = amax / Fmax (IEEE division); 1 for an all-zero
// tensor; NaN (canonical) when the tensor holds a NaN.
template <int FMT>
__device__ __forceinline__ float tensor_scale_from_key(uint32_t key)
{
    if (key > 0x7F800000u) return __uint_as_float(0x7FC00000u);
    if (key == 0) return 1.0f;
    return __uint_as_float(key) / Fmt<FMT>::fmax;
}

template <int FMT>
__device__ __forceinline__ float load_tensor_scale(const QArgs& a)
{
    if (a.two_level == 1) return tensor_scale_from_key<FMT>(*(const uint32_t*)a.tscale);
    return *a.tscale;
}

// code for an element of a NaN/Inf block: the format's NaN with the
// element's sign (FP8), 0 (FP4, which has no NaN)
template <int FMT>
__device__ __forceinline__ uint32_t nan_code(float v)
{
    if constexpr (FMT == E2M1) return 0u;
    return 0x7Fu | ((__float_as_uint(v) >> 24) & 0x80u);
}

template <int SRC, int FMT, bool ROW, bool COL>
__global__ __launch_bounds__(256) void k_quant(QArgs a)
{
    constexpr int W = kSubW;
    constexpr int BITS = Fmt<FMT>::bits;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t r0 = ((int64_t)blockIdx.y * kWaves + wave) * 32;
    if (r0 >= a.rows) return;                       // no LDS / barriers in this kernel
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * W;
    const int ncol = c0 < a.cols ? (int)(a.cols - c0 < W ? a.cols - c0 : W) : 0;
    const int nrow = (int)(a.rows - r0 < 32 ? a.rows - r0 : 32);

    // ---- load the 32 x W sub-tile (zero outside the tensor) ----
    float v[32][W];
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const int64_t base = (r0 + i) * a.ld + c0;
        if (i < nrow && ncol == W) {
            if constexpr (SRC == SRC_BF16) {
                const uint2 w = *(const uint2*)((const uint16_t*)a.x + base);
                v[i][0] = bf16_lo(w.x); v[i][1] = bf16_hi(w.x);
                v[i][2] = bf16_lo(w.y); v[i][3] = bf16_hi(w.y);
            } else {
                const float4 w = *(const float4*)((const float*)a.x + base);
                v[i][0] = w.x; v[i][1] = w.y; v[i][2] = w.z; v[i][3] = w.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < W; j++) {
                float t = 0.0f;
                if (i < nrow && j < ncol) {
                    if constexpr (SRC == SRC_BF16) t = __uint_as_float((uint32_t)((const uint16_t*)a.x)[base + j] << 16);
                    else t = ((const float*)a.x)[base + j];
                }
                v[i][j] = t;
            }
        }
    }

    // ---- level 1 of the two-level scheme: x / s_t ----
    if (a.two_level) {
        const float st = load_tensor_scale<FMT>(a);
#pragma unroll
        for (int i = 0; i < 32; i++)
#pragma unroll
            for (int j = 0; j < W; j++) v[i][j] = v[i][j] / st;
    }

    // ---- row copy: 1x32 blocks spread over 8 lanes ----
    if constexpr (ROW) {
        const int64_t row_bytes = a.cols * BITS / 8;
        const int64_t nblk = a.cols / 32;
#pragma unroll
        for (int i = 0; i < 32; i++) {
            if (i >= nrow) continue;                     // wave-uniform
            float t[W];
#pragma unroll
            for (int j = 0; j < W; j++) t[j] = v[i][j];
            if (a.hadamard) {
                // stages h = 1, 2 inside the lane, h = 4, 8, 16 across lanes
#pragma unroll
                for (int st = 0; st < 2; st++) {         // W = 4: h = 1, 2
                    const int h = 1 << st;
#pragma unroll
                    for (int j = 0; j < W; j++)
                        if ((j & h) == 0) {
                            const float p = t[j], q = t[j + h];
                            t[j] = p + q;
                            t[j + h] = p - q;
                        }
                }
#pragma unroll
                for (int st = 0; st < 3; st++) {         // h = 4, 8, 16: lanes ^1, ^2, ^4
                    const int m = 1 << st;
#pragma unroll
                    for (int j = 0; j < W; j++) {
                        const float p = __shfl_xor(t[j], m);
                        t[j] = (lane & m) ? (p - t[j]) : (t[j] + p);
                    }
                }
            }
            uint32_t key = 0;
#pragma unroll
            for (int j = 0; j < W; j++) key = max(key, abs_key(t[j]));
            key = max(key, (uint32_t)__shfl_xor((int)key, 1));
            key = max(key, (uint32_t)__shfl_xor((int)key, 2));
            key = max(key, (uint32_t)__shfl_xor((int)key, 4));
            const bool finite = key < 0x7F800000u;
            const int e = finite ? block_exponent<FMT>(key) : 0;
            float y[W];
#pragma unroll
            for (int j = 0; j < W; j++) y[j] = scale_by(t[j], e);
            if (a.sr) {
                const uint64_t idx = (uint64_t)(r0 + i) * (uint64_t)a.cols + (uint64_t)c0;
                const u32x4 w = philox_block(idx >> 2, 0u, a.offset, a.k0, a.k1);  // cols % 4 == 0
                y[0] = sr_value<FMT>(y[0], w.x); y[1] = sr_value<FMT>(y[1], w.y);
                y[2] = sr_value<FMT>(y[2], w.z); y[3] = sr_value<FMT>(y[3], w.w);
            } else {
#pragma unroll
                for (int j = 0; j < W; j++) y[j] = clamp_fmax<FMT>(y[j]);
            }
            if (ncol == W) {
                uint8_t* dst = a.q_row + (r0 + i) * row_bytes + c0 * BITS / 8;
                if constexpr (BITS == 8) {
                    uint32_t packed = cvt2_fp8<FMT>(y[0], y[1]) | (cvt2_fp8<FMT>(y[2], y[3]) << 16);
                    if (!finite)
                        packed = nan_code<FMT>(t[0]) | (nan_code<FMT>(t[1]) << 8) |
                                 (nan_code<FMT>(t[2]) << 16) | (nan_code<FMT>(t[3]) << 24);
                    *(uint32_t*)dst = packed;
                } else {
                    uint32_t packed = cvt2_fp4(y[0], y[1]) | (cvt2_fp4(y[2], y[3]) << 8);
                    if (!finite) packed = 0;
                    *(uint16_t*)dst = (uint16_t)packed;
                }
                if ((lane & 7) == 0)
                    a.s_row[(r0 + i) * nblk + c0 / 32] = (uint8_t)(finite ? e + 127 : 0xFF);
            }
        }
    }

    // ---- column copy: 32x1 blocks inside the lane, stored transposed ----
    if constexpr (COL) {
        if (ncol == 0) return;
        if (a.hadamard) {
#pragma unroll
            for (int j = 0; j < W; j++) {
                float col[32];
#pragma unroll
                for (int i = 0; i < 32; i++) col[i] = v[i][j];
                fwht32(col);
#pragma unroll
                for (int i = 0; i < 32; i++) v[i][j] = col[i];
            }
        }
        int e[W];
        bool finite[W];
#pragma unroll
        for (int j = 0; j < W; j++) {
            uint32_t key = 0;
#pragma unroll
            for (int i = 0; i < 32; i++) key = max(key, abs_key(v[i][j]));
            finite[j] = key < 0x7F800000u;
            e[j] = finite[j] ? block_exponent<FMT>(key) : 0;
        }
        // codes of column j, element i at byte i (FP8) / nibble i (FP4)
        constexpr int NW = BITS == 8 ? 8 : 4;           // dwords per column block
        uint32_t code[W][NW];
#pragma unroll
        for (int j = 0; j < W; j++)
#pragma unroll
            for (int k = 0; k < NW; k++) code[j][k] = 0;
        const bool fast_rng = (a.cols % 4) == 0;
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
            float y[2][W];
#pragma unroll
            for (int d = 0; d < 2; d++)
#pragma unroll
                for (int j = 0; j < W; j++) y[d][j] = scale_by(v[i + d][j], e[j]);
            if (a.sr) {
#pragma unroll
                for (int d = 0; d < 2; d++) {
                    const uint64_t idx = (uint64_t)(r0 + i + d) * (uint64_t)a.cols + (uint64_t)c0;
                    if (fast_rng) {
                        const u32x4 w = philox_block(idx >> 2, 1u, a.offset, a.k0, a.k1);
                        y[d][0] = sr_value<FMT>(y[d][0], w.x); y[d][1] = sr_value<FMT>(y[d][1], w.y);
                        y[d][2] = sr_value<FMT>(y[d][2], w.z); y[d][3] = sr_value<FMT>(y[d][3], w.w);
                    } else {
#pragma unroll
                        for (int j = 0; j < W; j++) {
                            const uint64_t ij = idx + j;
                            const u32x4 w = philox_block(ij >> 2, 1u, a.offset, a.k0, a.k1);
                            y[d][j] = sr_value<FMT>(y[d][j], pick(w, (uint32_t)(ij & 3)));
                        }
                    }
                }
            } else {
#pragma unroll
                for (int d = 0; d < 2; d++)
#pragma unroll
                    for (int j = 0; j < W; j++) y[d][j] = clamp_fmax<FMT>(y[d][j]);
            }
#pragma unroll
            for (int j = 0; j < W; j++) {
                if constexpr (BITS == 8) {
                    uint32_t c2 = cvt2_fp8<FMT>(y[0][j], y[1][j]);
                    if (!finite[j]) c2 = nan_code<FMT>(v[i][j]) | (nan_code<FMT>(v[i + 1][j]) << 8);
                    code[j][i / 4] |= c2 << (8 * (i % 4));
                } else {
                    uint32_t c2 = cvt2_fp4(y[0][j], y[1][j]);
                    if (!finite[j]) c2 = 0;
                    code[j][i / 8] |= c2 << (4 * (i % 8));
                }
            }
        }
        const int64_t col_bytes = a.rows * BITS / 8;
        const int64_t nblk = a.rows / 32;
#pragma unroll
        for (int j = 0; j < W; j++) {
            if (j < ncol) {
                uint8_t* dst = a.q_col + (c0 + j) * col_bytes + r0 * BITS / 8;
                *(uint4*)dst = make_uint4(code[j][0], code[j][1], code[j][2], code[j][3]);
                if constexpr (BITS == 8)
                    *(uint4*)(dst + 16) = make_uint4(code[j][4], code[j][5], code[j][6], code[j][7]);
                a.s_col[(c0 + j) * nblk + r0 / 32] = (uint8_t)(finite[j] ? e[j] + 127 : 0xFF);
            }
        }
    }
}

// ---- level-1 tensor amax: |x| keys reduced with an integer max ----
__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

template <int SRC>
__global__ __launch_bounds__(256) void k_amax(const void* x, int64_t rows, int64_t cols,
                                              int64_t ld, uint32_t* out)
{
    constexpr int W = 4;
    const int64_t chunks_per_row = (cols + W - 1) / W;
    const int64_t total = rows * chunks_per_row;
    uint32_t key = 0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / chunks_per_row;
        const int64_t c = (t - r * chunks_per_row) * W;
        const int64_t base = r * ld + c;
        if (c + W <= cols) {
            if constexpr (SRC == SRC_BF16) {
                const uint2 w = *(const uint2*)((const uint16_t*)x + base);
                key = max(key, max(max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu),
                                   max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu)) << 16);
            } else {
                const uint4 w = *(const uint4*)((const float*)x + base);
                key = max(key, max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu),
                                   max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu)));
            }
        } else {
            for (int64_t j = c; j < cols; j++) {
                uint32_t b;
                if constexpr (SRC == SRC_BF16) b = (uint32_t)((const uint16_t*)x)[r * ld + j] << 16;
                else b = ((const uint32_t*)x)[r * ld + j];
                key = max(key, b & 0x7FFFFFFFu);
            }
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t k = max(max(red[0], red[1]), max(red[2], red[3]));
        atomicMax(out, k);
    }
}

template <int FMT>
__global__ void k_tscale_finalize(float* ts)
{
    const uint32_t key = *(const uint32_t*)ts;
    *ts = tensor_scale_from_key<FMT>(key);
}

template <int SRC, int FMT>
hipError_t launch_fmt(const QuantJob& j, hipStream_t stream)
{
    QArgs a;
    a.x = j.x; a.rows = j.rows; a.cols = j.cols; a.ld = j.ld;
    a.q_row = j.q_row; a.s_row = j.s_row; a.q_col = j.q_col; a.s_col = j.s_col;
    a.tscale = j.tensor_scale;
    a.k0 = (uint32_t)j.seed; a.k1 = (uint32_t)(j.seed >> 32); a.offset = j.offset;
    a.sr = j.sr; a.hadamard = j.hadamard; a.two_level = j.two_level;

    if (j.two_level == 1) {
        uint32_t* word = (uint32_t*)j.tensor_scale;
        k_fill_u32<<<1, 1, 0, stream>>>(word, 0u);
        const int64_t chunks = j.rows * ((j.cols + 3) / 4);
        int64_t blocks = (chunks + 255) / 256;
        if (blocks > 1024) blocks = 1024;
        k_amax<SRC><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(j.x, j.rows, j.cols, j.ld, word);
    }
    const dim3 grid((unsigned)((j.cols + 64 * kSubW - 1) / (64 * kSubW)),
                    (unsigned)((j.rows + 32 * kWaves - 1) / (32 * kWaves)));
    const dim3 block(256);
    if (j.q_row && j.q_col) k_quant<SRC, FMT, true, true><<<grid, block, 0, stream>>>(a);
    else if (j.q_row) k_quant<SRC, FMT, true, false><<<grid, block, 0, stream>>>(a);
    else k_quant<SRC, FMT, false, true><<<grid, block, 0, stream>>>(a);
    if (j.two_level == 1) k_tscale_finalize<FMT><<<1, 1, 0, stream>>>(j.tensor_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantJob& j, hipStream_t stream)
{
    const bool bf = j.src == SRC_BF16;
    switch (j.fmt) {
    case E4M3: return bf ? launch_fmt<SRC_BF16, E4M3>(j, stream) : launch_fmt<SRC_F32, E4M3>(j, stream);
    case E5M2: return bf ? launch_fmt<SRC_BF16, E5M2>(j, stream) : launch_fmt<SRC_F32, E5M2>(j, stream);
    default:   return bf ? launch_fmt<SRC_BF16, E2M1>(j, stream) : launch_fmt<SRC_F32, E2M1>(j, stream);
    }
}

}  // namespace mx
