// dequant.hip -- MX dequantization for gfx950 ([MOSS, "两级缩放实现"]:
// the micro-scale is undone first, then the tensor scale; the power-of-two
// micro-scale makes the first step an exact exponent shift, [MOSS,
// "Power-of-Two 的关键优势"]).  Per block: decode(code) * 2^(byte-127) exactly
// in fp32, then the inverse fixed-sign Hadamard (FWHT * 1/32) if the copy was
// quantized with it, then one fp32 multiply by the tensor scale.  Output in
// the source layout.
//
// Sources:
//   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
//
// One thread per 32-element block.  Row copies: consecutive threads take
// consecutive blocks of a row (each writes 32 contiguous outputs).  Column
// copies: consecutive threads take consecutive columns, so every output row
// is written by a wave as one contiguous run.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

template <int FMT>
__device__ __forceinline__ float decode(uint32_t c)
{
    constexpr int E = FMT == E4M3 ? 4 : FMT == E5M2 ? 5 : 2;
    constexpr int M = Fmt<FMT>::mbits;
    constexpr int B = FMT == E4M3 ? 7 : FMT == E5M2 ? 15 : 1;
    const uint32_t s = (c >> (E + M)) & 1u;
    const uint32_t e = (c >> M) & ((1u << E) - 1u);
    const uint32_t m = c & ((1u << M) - 1u);
    float v;
    if (FMT == E4M3 && e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
    else if (FMT == E5M2 && e == 31) v = m == 0 ? __uint_as_float(0x7F800000u) : __uint_as_float(0x7FC00000u);
    else if (e == 0) v = (float)m * exp2i(1 - B - M);                  // subnormal: exact
    else v = __uint_as_float(((e - B + 127) << 23) | (m << (23 - M)));  // normal: exact
    return s ? -v : v;
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f)
{
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);  // quiet NaN
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <int FMT, int AXIS, int OUT, bool HAD, bool TS>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ ts, int64_t rows,
                                                 int64_t cols, void* __restrict__ out)
{
    constexpr int BITS = Fmt<FMT>::bits;
    // stored copy: [orows][ocols]; blocks along ocols
    const int64_t orows = AXIS == 0 ? rows : cols;
    const int64_t ocols = AXIS == 0 ? cols : rows;
    const int64_t nblk = ocols / 32;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= orows * nblk) return;
    int64_t orow, oblk;
    if (AXIS == 0) { orow = t / nblk; oblk = t - orow * nblk; }     // blocks of a row adjacent
    else { oblk = t / orows; orow = t - oblk * orows; }              // columns adjacent
    const uint8_t* src = q + orow * (ocols * BITS / 8) + oblk * 32 * BITS / 8;
    uint32_t w[8];
    const uint4 lo = *(const uint4*)src;
    w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
    if constexpr (BITS == 8) {
        const uint4 hi = *(const uint4*)(src + 16);
        w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    }
    const uint32_t sb = scales[orow * nblk + oblk];
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint32_t c = BITS == 8 ? (w[i / 4] >> (8 * (i % 4))) & 0xFFu
                                     : (w[i / 8] >> (4 * (i % 8))) & 0xFu;
        const float d = decode<FMT>(c);
        v[i] = sb == 0xFFu ? __uint_as_float(0x7FC00000u) : ldexpf(d, (int)sb - 127);
    }
    if constexpr (HAD) {
        fwht32(v);
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = v[i] * 0.03125f;
    }
    if constexpr (TS) {
        const float s = *ts;
#pragma unroll
        for (int i = 0; i < 32; i++) v[i] = v[i] * s;
    }
    if constexpr (AXIS == 0) {
        const int64_t base = orow * cols + oblk * 32;
        if constexpr (OUT == 0) {
            float4* o = (float4*)((float*)out + base);
#pragma unroll
            for (int k = 0; k < 8; k++) o[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
        } else {
            uint4* o = (uint4*)((uint16_t*)out + base);
#pragma unroll
            for (int k = 0; k < 4; k++) {
                uint32_t p[4];
#pragma unroll
                for (int h = 0; h < 4; h++)
                    p[h] = (uint32_t)to_bf16_rne(v[8 * k + 2 * h]) | ((uint32_t)to_bf16_rne(v[8 * k + 2 * h + 1]) << 16);
                o[k] = make_uint4(p[0], p[1], p[2], p[3]);
            }
        }
    } else {
        const int64_t c = orow, r0 = oblk * 32;
#pragma unroll
        for (int i = 0; i < 32; i++) {
            if constexpr (OUT == 0) ((float*)out)[(r0 + i) * cols + c] = v[i];
            else ((uint16_t*)out)[(r0 + i) * cols + c] = to_bf16_rne(v[i]);
        }
    }
}

template <int FMT, int AXIS, int OUT>
hipError_t launch3(const DequantJob& j, hipStream_t s)
{
    const int64_t nthreads = j.rows * j.cols / 32;
    const dim3 grid((unsigned)((nthreads + 255) / 256)), block(256);
    const bool ts = j.tensor_scale != nullptr;
    if (j.hadamard) {
        if (ts) k_dequant<FMT, AXIS, OUT, true, true><<<grid, block, 0, s>>>(j.q, j.scales, j.tensor_scale, j.rows, j.cols, j.out);
        else k_dequant<FMT, AXIS, OUT, true, false><<<grid, block, 0, s>>>(j.q, j.scales, j.tensor_scale, j.rows, j.cols, j.out);
    } else {
        if (ts) k_dequant<FMT, AXIS, OUT, false, true><<<grid, block, 0, s>>>(j.q, j.scales, j.tensor_scale, j.rows, j.cols, j.out);
        else k_dequant<FMT, AXIS, OUT, false, false><<<grid, block, 0, s>>>(j.q, j.scales, j.tensor_scale, j.rows, j.cols, j.out);
    }
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const DequantJob& j, hipStream_t s)
{
    if (j.axis == 0) return j.out_dtype == 0 ? launch3<FMT, 0, 0>(j, s) : launch3<FMT, 0, 1>(j, s);
    return j.out_dtype == 0 ? launch3<FMT, 1, 0>(j, s) : launch3<FMT, 1, 1>(j, s);
}

}  // namespace

hipError_t launch_dequantize(const DequantJob& j, hipStream_t stream)
{
    switch (j.fmt) {
    case E4M3: return launch_fmt<E4M3>(j, stream);
    case E5M2: return launch_fmt<E5M2>(j, stream);
    default: return launch_fmt<E2M1>(j, stream);
    }
}

}  // namespace mx
