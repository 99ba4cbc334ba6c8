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
#include <algorithm>

#include <type_traits>

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

// 8 consecutive source elements from x[i] (16-byte aligned) as floats
template <int SRC> __device__ __forceinline__ void load8(const void* x, int64_t i, float* v)
{
    if constexpr (SRC == SRC_BF16) {
        const uint4 u = *(const uint4*)((const uint16_t*)x + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *(const float4*)((const float*)x + i), b = *(const float4*)((const float*)x + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// x[r][c0 .. c0+7] (zero past `cols`), vectorized when `vec` (16-byte
// aligned rows, cols % 8 == 0)
template <int SRC>
__device__ __forceinline__ void row8(const void* x, int64_t ld, int64_t cols, bool vec, int64_t r, int64_t c0, float* v)
{
    if (vec && c0 + 8 <= cols) {
        load8<SRC>(x, r * ld + c0, v);
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = c0 + k < cols ? src_at<SRC>(x, r * ld + c0 + k) : 0.0f;
    }
}

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// second-level scale of a domain from its amax key: NaN for a NaN or Inf, 1
// for an all-zero domain, else amax / (6 * 448)
__device__ __forceinline__ float domain_scale(uint32_t key)
{
    return key >= 0x7F800000u ? __builtin_nanf("") : key == 0 ? 1.0f : __uint_as_float(key) / 2688.0f;
}

// ---------------------------------------------------------------------------
// second-level scales: per-panel amax partials, then the scales
// ---------------------------------------------------------------------------
// Element tiles are 32 source rows x 256 source columns.  A panel (32
// stored rows) is a tile row of the source for the row copy and eight
// consecutive 32-column strips for the column copy.  Workgroup (a, g) takes
// tile a across the panels and S consecutive tiles along them (tiles
// g*S ..), reducing to one amax key per panel it touches:
//   row copy:    partial[a * G + g]             (panel a)
//   column copy: partial[(8 a + k) * G + g]     (panels 8a + k, k < 8)
// Thread t reads 8 columns (chunk t % 32) of rows t / 32 + 8 i, i < 4, of a
// tile: 16- or 32-byte loads, 128 contiguous bytes per wave row.
template <int SRC, bool ROW>
__global__ __launch_bounds__(256) void k_nv_amax(const void* x, int64_t rows, int64_t cols, int64_t ld, bool vec,
                                                 int tiles_across, int tiles_along, int S, int G, int64_t npanels,
                                                 uint32_t* partial)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, cc = t & 31;
    __shared__ uint32_t red[4][8];
    for (int64_t w = blockIdx.x; w < (int64_t)tiles_across * G; w += gridDim.x) {
        const int a = (int)(w / G), g = (int)(w % G);
        uint32_t key = 0;
        for (int e = g * S; e < min(g * S + S, tiles_along); e++) {
            const int tr = ROW ? a : e, tc = ROW ? e : a;
            const int64_t c0 = (int64_t)tc * 256 + 8 * cc;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t r = (int64_t)tr * 32 + (t >> 5) + 8 * i;
                if (r < rows && c0 < cols) {
                    float v[8];
                    row8<SRC>(x, ld, cols, vec, r, c0, v);
#pragma unroll
                    for (int k = 0; k < 8; k++) key = max(key, abs_bits(v[k]));
                }
            }
        }
        if (ROW) {                                   // one panel: the whole workgroup
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
            if (lane == 0) red[wave][0] = key;
            __syncthreads();
            if (t == 0) partial[(int64_t)a * G + g] = max(max(red[0][0], red[1][0]), max(red[2][0], red[3][0]));
        } else {                                     // panel of chunk cc: 8 a + cc / 4
            key = max(key, (uint32_t)__shfl_xor((int)key, 1));
            key = max(key, (uint32_t)__shfl_xor((int)key, 2));
            key = max(key, (uint32_t)__shfl_xor((int)key, 32));
            if (lane < 32 && (lane & 3) == 0) red[wave][lane >> 2] = key;
            __syncthreads();
            if (t < 8) {
                const int64_t p = 8 * (int64_t)a + t;
                if (p < npanels) partial[p * G + g] = max(max(red[0][t], red[1][t]), max(red[2][t], red[3][t]));
            }
        }
        __syncthreads();
    }
}

// CTA-local: ts[p] from the G partials of panel p
__global__ __launch_bounds__(256) void k_nv_scales_local(const uint32_t* partial, int64_t npanels, int G, float* ts)
{
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < npanels; p += (int64_t)gridDim.x * 256) {
        uint32_t key = 0;
        for (int g = 0; g < G; g++) key = max(key, partial[p * G + g]);
        ts[p] = domain_scale(key);
    }
}

// global: ts[0] from all n partials, one workgroup
__global__ __launch_bounds__(1024) void k_nv_scale_global(const uint32_t* partial, int64_t n, float* ts)
{
    uint32_t key = 0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) key = max(key, partial[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    __shared__ uint32_t red[16];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < 16; i++) key = max(key, red[i]);
        ts[0] = domain_scale(key);
    }
}

// ---------------------------------------------------------------------------
// quantize
// ---------------------------------------------------------------------------
// one block of 16 values under second-level scale s: returns the E4M3
// scale byte, writes the 16 E2M1 codes (element 2j in the low nibble of
// byte j) to w[0..1]
__device__ __forceinline__ uint32_t nv_block(const float* v, float s, uint32_t* w)
{
    uint32_t key = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) key = max(key, abs_bits(v[i]));
    w[0] = w[1] = 0;
    if (key >= 0x7F800000u || s != s) return 0x7Fu;
    const float den = 6.0f * s;
    const float bv = __uint_as_float(key) / den;
    const uint32_t sb = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fmax<E4M3>(bv), 0.0f, 0, false) & 0x7Fu;
    const float ds = e4m3_value(sb);
    if (ds == 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; i++) w[0] |= (__float_as_uint(v[i]) >> 31) << (4 * i + 3);
#pragma unroll
        for (int i = 0; i < 8; i++) w[1] |= (__float_as_uint(v[8 + i]) >> 31) << (4 * i + 3);
    } else {
        const float d = ds * s;
        const float r = 1.0f / d;
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; i++) y[i] = clamp_fmax<E2M1>(v[i] * r);
        w[0] = cvt8_fp4(y);
        w[1] = cvt8_fp4(y + 8);
    }
    return sb;
}

// row copy: one thread per block of 16 along the source row; consecutive
// threads take consecutive blocks (32- or 64-byte loads)
template <int SRC>
__global__ __launch_bounds__(256) void k_nv_quant_row(const void* x, int64_t rows, int64_t cols, int64_t ld, bool vec,
                                                      int local, const float* ts, uint8_t* q, uint8_t* s16)
{
    const int64_t nb = cols / 16, total = rows * nb;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t r = t / nb, b = t % nb;
        float v[16];
        row8<SRC>(x, ld, cols, vec, r, b * 16, v);
        row8<SRC>(x, ld, cols, vec, r, b * 16 + 8, v + 8);
        uint32_t w[2];
        const uint32_t sb = nv_block(v, ts[local ? r / NV_PANEL : 0], w);
        s16[t] = (uint8_t)sb;
        *(uint2*)(q + r * (cols / 2) + b * 8) = make_uint2(w[0], w[1]);
    }
}

// column copy: tiles of 128 source rows x 64 source columns staged through
// LDS (fp32, rows padded to 65).  Loads: 8 columns of a row per thread per
// step, rows of 128 contiguous bytes (bf16).  Quantization: thread t takes
// column t / 4 and its blocks 2 (t % 4) and 2 (t % 4) + 1, so four
// consecutive lanes write one stored row's 64 contiguous code bytes.
template <int SRC>
__global__ __launch_bounds__(256) void k_nv_quant_col(const void* x, int64_t rows, int64_t cols, int64_t ld, bool vec,
                                                      int local, const float* ts, uint8_t* q, uint8_t* s16)
{
    constexpr int TR = 128, TC = 64, PAD = TC + 1;
    __shared__ float tile[TR * PAD];
    const int t = threadIdx.x;
    const int64_t tiles_r = (rows + TR - 1) / TR, tiles_c = (cols + TC - 1) / TC;
    const int64_t nb = rows / 16;                    // blocks per stored row
    for (int64_t w = blockIdx.x; w < tiles_r * tiles_c; w += gridDim.x) {
        const int64_t r0 = (w / tiles_c) * TR, c0 = (w % tiles_c) * TC;
        // 128 rows x 8 chunks of 8 columns: 4 per thread
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int id = t + 256 * i, rr = id >> 3, ch = id & 7;
            const int64_t r = r0 + rr, c = c0 + 8 * ch;
            float v[8];
            if (r < rows && c < cols) row8<SRC>(x, ld, cols, vec, r, c, v);
            else {
#pragma unroll
                for (int k = 0; k < 8; k++) v[k] = 0.0f;
            }
#pragma unroll
            for (int k = 0; k < 8; k++) tile[rr * PAD + 8 * ch + k] = v[k];
        }
        __syncthreads();
        const int cl = t >> 2, bp = t & 3;
        const int64_t sr = c0 + cl;                  // stored row = source column
        if (sr < cols) {
            const float s = ts[local ? sr / NV_PANEL : 0];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int blk = 2 * bp + h;          // block within the tile (rows 16 blk ..)
                const int64_t bi = r0 / 16 + blk;    // block within the stored row
                if (bi < nb) {
                    float v[16];
#pragma unroll
                    for (int i = 0; i < 16; i++) v[i] = tile[(16 * blk + i) * PAD + cl];
                    uint32_t wq[2];
                    const uint32_t sb = nv_block(v, s, wq);
                    s16[sr * nb + bi] = (uint8_t)sb;
                    *(uint2*)(q + sr * (rows / 2) + bi * 8) = make_uint2(wq[0], wq[1]);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// k_nv_quant_local: the CTA-local route in one pass.  One 1024-thread
// workgroup per panel of 32 stored rows of a bf16 source whose blocked
// length L is at most 4096: the panel (32 x L elements, at most 256 KiB) is
// read once into registers (16 bytes x 16 per thread), its amax reduced
// inside the workgroup into the panel's scale, and its blocks quantized from
// the registers.  No other workgroup is involved, so there is no second
// kernel and no second read of the source.
//   row copy (panel = source rows 32p..): thread chunk c = tid + 1024 i is
//     8 consecutive elements of panel row c / (L / 8); the two threads
//     holding a 16-block (adjacent lanes) exchange their maxima by a lane
//     shuffle and each writes its 8 codes (4 bytes).
//   column copy (panel = source columns 32p..): thread tid holds row block
//     tid / 4 (16 source rows) x column group tid % 4 (8 columns), i.e. 8
//     whole column blocks; four adjacent lanes read a row's 64-byte panel
//     segment, and 16 lanes write 128 contiguous code bytes of a column.
// ---------------------------------------------------------------------------
constexpr int NV_FUSED_THREADS = 1024, NV_FUSED_MAXL = 4096;

// E4M3 block-scale byte and the code reciprocal r of a block whose amax key
// is `key` under the panel's second-level scale s -- the arithmetic of
// nv_block (a zero scale gives r = 0: signed-zero codes; a NaN block or
// domain 0x7F) with the panel's divisions hoisted: amax / (6 s) through
// the reciprocal-plus-residual division (the IEEE quotient; IEEE division
// outside its range), and RN(1 / RN(decode(sb) s)) from a table of the 127
// finite scale codes -- the same values, computed once per panel
__device__ __forceinline__ uint32_t nv_block_scale_tab(uint32_t key, float s, const TensorDiv& dden,
                                                       const float* rtab, float& r)
{
    r = 0.0f;
    if (key >= 0x7F800000u || s != s) return 0x7Fu;
    const float a = __uint_as_float(key);
    uint32_t lo = ~0u;
    float bv = div_fast(a, dden, lo);
    if (!dden.fast || lo < dden.lo_key || bv > 0x1p17f) bv = a / dden.s;
    const uint32_t sb = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fmax<E4M3>(bv), 0.0f, 0, false) & 0x7Fu;
    r = rtab[sb];
    return sb;
}

// 8 codes of 8 bf16 values (packed in 4 dwords) under a block scale: r = 0
// gives the signed zeros, sb = 0x7F zero codes
__device__ __forceinline__ uint32_t nv_encode8(const uint32_t* w, uint32_t sb, float r)
{
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        y[2 * k] = __uint_as_float(w[k] << 16);
        y[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
    if (sb == 0x7Fu) return 0u;
    if (r == 0.0f) {
        uint32_t z = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) z |= (__float_as_uint(y[i]) >> 31) << (4 * i + 3);
        return z;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = clamp_fmax<E2M1>(y[i] * r);
    return cvt8_fp4(y);
}

// |max| key of 8 bf16 values packed in 4 dwords (NaN above Inf above finite)
__device__ __forceinline__ uint32_t bf16x8_key(const uint32_t* w)
{
    uint32_t key = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) key = max(key, max((w[k] & 0x7FFFu) << 16, w[k] & 0x7FFF0000u));
    return key;
}

// ---------------------------------------------------------------------------
// k_nv_quant_local: the CTA-local route in one pass.  One 1024-thread
// workgroup per panel of 32 stored rows of a bf16 source whose blocked
// length L is at most 4096: the panel (32 x L elements, at most 256 KiB) is
// read once into registers (16 bytes x 16 per thread), its amax reduced
// inside the workgroup into the panel's scale, and its blocks quantized from
// the registers.  No other workgroup is involved, so there is no second
// kernel and no second read of the source.
//   row copy (panel = source rows 32p..): thread chunk c = tid + 1024 i is
//     8 consecutive elements of panel row c / (L / 8); the two threads
//     holding a 16-block (adjacent lanes) exchange their maxima by a lane
//     shuffle and each writes its 8 codes (4 bytes).
//   column copy (panel = source columns 32p..): thread tid holds row block
//     tid / 4 (16 source rows) x column group tid % 4 (8 columns), i.e. 8
//     whole column blocks; four adjacent lanes read a row's 64-byte panel
//     segment, and 16 lanes write 128 contiguous code bytes of a column.
// ---------------------------------------------------------------------------
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t nv_rsrc(const void* base, int64_t bytes)
{
    bytes = bytes < 0 ? 0 : bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

template <bool ROW>
__global__ __launch_bounds__(1024) void k_nv_quant_local(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                                         int64_t npanels, float* ts, uint8_t* q, uint8_t* s16)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t L = ROW ? cols : rows, SR = ROW ? rows : cols, nb = L / 16;
    const int cpr = (int)(L / 8);                    // row copy: 8-element chunks per panel row
    const int nrb = (int)(L / 16);                   // column copy: 16-row blocks
    __shared__ uint32_t red[16];
    __shared__ float panel_s;
    __shared__ float rtab[128];                      // RN(1 / RN(e4m3(c) s)), 0 for a zero scale
    for (int64_t w = blockIdx.x; w < npanels; w += gridDim.x) {
        // Column copy: a panel's rows are 64-byte halves of 128-byte lines whose
        // other halves belong to the neighbouring panels.  Workgroups are dealt
        // to the 8 XCDs round-robin; giving each XCD a contiguous range of
        // panels (when the grid is one panel per workgroup and divides by 8)
        // lets neighbours share their lines in one L2 instead of fetching them
        // twice from HBM.
        const int64_t p = (!ROW && gridDim.x == npanels && (npanels & 7) == 0)
                              ? (w & 7) * (npanels >> 3) + (w >> 3) : w;
        // the thread index passes through an empty asm per panel, so that the
        // 16 load offsets are recomputed here rather than hoisted out of the
        // panel loop (where they would stay live, and spill, beside the data)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int64_t sr0 = p * NV_PANEL;
        const int np = (int)min((int64_t)NV_PANEL, SR - sr0);      // stored rows in this panel
        // buffer views of the panel: 32-bit offsets; source rows / stored rows
        // past the panel read as zero and their stores are dropped
        const auto rx = ROW ? nv_rsrc(x + sr0 * ld, ((int64_t)(np - 1) * ld + L) * 2)
                            : nv_rsrc(x + sr0, ((L - 1) * ld + (SR - sr0)) * 2);
        const auto rq = nv_rsrc(q + sr0 * (L / 2), (int64_t)np * (L / 2));
        const auto rs = nv_rsrc(s16 + sr0 * nb, (int64_t)np * nb);
        uint4 v[16];
        if (ROW) {
            // thread: panel row tid / 32, chunks (tid % 32) + 32 i
            const int r = tid >> 5;
            const uint32_t base = (uint32_t)((int64_t)r * ld * 2) + (uint32_t)((tid & 31) * 16);
#pragma unroll
            for (int i = 0; i < 16; i++) {
                // chunks past the row (L < 4096) get an offset at or above 2^31
                const uint32_t off = base + (uint32_t)(512 * i) + ((tid & 31) + 32 * i < cpr ? 0u : 0x80000000u);
                v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            }
        } else {
            // unit: row block tid / 4, column group tid % 4 -- four adjacent
            // lanes read one row's 64-byte panel segment
            const int rb = tid >> 2, cg = tid & 3;
            // a unit past the panel (SR % 8 == 0 here: whole chunks) gets an
            // offset at or above 2^31, beyond the view's range (below 2^31)
            const uint32_t base = (uint32_t)(((int64_t)rb * 16 * ld + 8 * cg) * 2) +
                                  ((rb < nrb && 8 * cg < np) ? 0u : 0x80000000u);
            const uint32_t rstep = (uint32_t)(ld * 2);
#pragma unroll
            for (int i = 0; i < 16; i++)
                v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, base + (uint32_t)i * rstep, 0, 0));
        }
        // all 16 loads in flight before the first use
        __builtin_amdgcn_sched_barrier(0);
        // panel amax
        uint32_t key = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            key = max(key, bf16x8_key(w));
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
        if (lane == 0) red[wave] = key;
        __syncthreads();
        if (tid == 0) {
            uint32_t k2 = red[0];
            for (int i = 1; i < 16; i++) k2 = max(k2, red[i]);
            panel_s = domain_scale(k2);
            ts[p] = panel_s;
        }
        __syncthreads();
        const float s = panel_s;
        if (tid < 128) {
            const float ds = e4m3_value((uint32_t)tid);
            rtab[tid] = ds == 0.0f ? 0.0f : 1.0f / (ds * s);
        }
        const TensorDiv dden = make_div(6.0f * s);
        __syncthreads();
        // (likewise for the store offsets, and for the held data: nothing of
        // the quantization is computed before the panel's scale is known)
        asm volatile("" : "+v"(tid));
#pragma unroll
        for (int i = 0; i < 16; i++) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
        if (ROW) {
            const int r = tid >> 5;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                // chunks cc and cc ^ 1 (adjacent lanes) form one 16-block; every
                // lane takes part in the shuffle
                const int cc = (tid & 31) + 32 * i;
                const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                const uint32_t own = bf16x8_key(w);
                const uint32_t bkey = max(own, (uint32_t)__shfl_xor((int)own, 1));
                float rc;
                const uint32_t sb = nv_block_scale_tab(bkey, s, dden, rtab, rc);
                const uint32_t codes = nv_encode8(w, sb, rc);
                if (cc < cpr) {
                    const uint32_t qo = (uint32_t)(r * (L / 2) + (cc >> 1) * 8 + (cc & 1) * 4);
                    __builtin_amdgcn_raw_buffer_store_b32(codes, rq, qo, 0, 0);
                    if ((cc & 1) == 0) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, (uint32_t)(r * nb + (cc >> 1)), 0, 0);
                }
                // one chunk at a time: keeps the scheduler from overlapping the
                // chunks' temporaries with the 64 registers of held data
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const int rb = tid >> 2, cg = tid & 3;
            if (rb < nrb) {
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    // column k of the 16 rows, as two runs of 8 packed bf16
                    uint32_t lo[4], hi[4];
#pragma unroll
                    for (int i = 0; i < 8; i += 2) {
                        const uint32_t a0 = k < 2 ? v[i].x : k < 4 ? v[i].y : k < 6 ? v[i].z : v[i].w;
                        const uint32_t a1 = k < 2 ? v[i + 1].x : k < 4 ? v[i + 1].y : k < 6 ? v[i + 1].z : v[i + 1].w;
                        const uint32_t b0 = k < 2 ? v[8 + i].x : k < 4 ? v[8 + i].y : k < 6 ? v[8 + i].z : v[8 + i].w;
                        const uint32_t b1 = k < 2 ? v[9 + i].x : k < 4 ? v[9 + i].y : k < 6 ? v[9 + i].z : v[9 + i].w;
                        // element k of a dword pair: low halves for even k, high for odd
                        lo[i / 2] = (k & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u) : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
                        hi[i / 2] = (k & 1) ? __builtin_amdgcn_perm(b1, b0, 0x07060302u) : __builtin_amdgcn_perm(b1, b0, 0x05040100u);
                    }
                    const uint32_t bkey = max(bf16x8_key(lo), bf16x8_key(hi));
                    float rc;
                    const uint32_t sb = nv_block_scale_tab(bkey, s, dden, rtab, rc);
                    const uint32_t c0 = nv_encode8(lo, sb, rc), c1 = nv_encode8(hi, sb, rc);
                    const int srl = 8 * cg + k;              // stored row within the panel
                    const uint32_t qo = (uint32_t)(srl * (L / 2) + rb * 8);
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2v{c0, c1}, rq, qo, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs, (uint32_t)(srl * nb + rb), 0, 0);
                }
            }
        }
        __syncthreads();                             // panel_s and red are reused by the next panel
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
// per 512-thread workgroup, K advancing 64 elements per stage.  Each stage's
// codes and block scales are dequantized exactly to f16 (converter with 2^E,
// packed multiply by the integer factor) into one of two LDS stage buffers
// (rows of 128 bytes whose 16-byte chunks are XOR-swizzled by
// (row >> 1) & 7, conflict-free for the fragment reads), and multiplied on
// the f16 matrix cores (32x32x16) with fp32 accumulation.
//
// Two waves per SIMD in two groups (waves 0-3 and 4-7; wave w runs on SIMD
// w % 4): each wave computes a 128x64 piece of its SIMD's 128x128 quarter.
// A stage takes two phases separated by workgroup barriers; in each, one
// group multiplies the stage from LDS while the other dequantizes its half
// of the next stage (A and B rows 128 g .. 128 g + 127 for group g) into
// the other buffer and loads its half of a later stage into registers.  The SIMD thus overlaps one wave's MFMAs with the other's
// conversions, LDS writes and loads (a probe: VALU work of one wave runs
// under another wave's MFMAs at no cost in cycles).  The second-level
// scales and alpha are applied once per output in the epilogue.
// ---------------------------------------------------------------------------
// workgroup barrier that waits for this wave's LDS traffic only (not for
// its global loads, which a fence-carrying __syncthreads would drain)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f16acc __attribute__((ext_vector_type(16)));

constexpr int NBM = 256, NBK = 64, NROWB = NBK * 2;   // tile rows, K per stage, f16 bytes per tile row

__device__ __forceinline__ int nv_swz(int row, int chunk) { return row * NROWB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// one 16-byte chunk of codes (32 elements, two blocks) and its two block
// scales -> 32 exact f16 values into LDS row `row`, chunks 4*half .. 4*half+3.
// Both converters are exact here: the FP4 one (scale 1) gives the E2M1
// values, the FP8 one gives the two E4M3 block scales (every E4M3 value,
// subnormals and NaN included, is an f16), and their product has at most
// 6 significant bits and lies in [2^-10, 2688] -- an f16, so the packed
// multiply does not round.
__device__ __forceinline__ void nv_dequant_chunk(uint8_t* tile, int row, int half, uint4 codes, uint32_t sc2)
{
    const h2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc2, 1.0f, false);   // {scale 0, scale 1}
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {                    // 16-byte output chunk q: code bytes 4q .. 4q+3
        const h2 f2 = q < 2 ? h2{sc[0], sc[0]} : h2{sc[1], sc[1]};   // bytes 0-7: block 0, 8-15: block 1
        const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 0) * f2;
        const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 1) * f2;
        const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 2) * f2;
        const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 3) * f2;
        *(h8*)(tile + nv_swz(row, 4 * half + q)) = h8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    }
}

template <int OUTT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_nv_gemm(NvGemmJob g, int tiles_m, int tiles_n)
{
    // stage buffer b: the A tile at b * 64 KiB, the B tile 32 KiB after it
    // (within reach of an LDS instruction's immediate offset)
    __shared__ __align__(16) uint8_t lds[2 * 2 * NBM * NROWB];
    auto tA = [&](int b) __attribute__((always_inline)) { return lds + b * (2 * NBM * NROWB); };
    auto tB = [&](int b) __attribute__((always_inline)) { return lds + b * (2 * NBM * NROWB) + NBM * NROWB; };
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, q = wave & 3;
    const int wm = q >> 1, wn = q & 1, h = lane >> 5, l32 = lane & 31;
    const int gt = tid & 255;                        // thread index inside the group

    // tile order: workgroups dealt round-robin to the 8 XCDs; each XCD takes a
    // contiguous range of tiles in row-major order of 4-row groups
    int t = blockIdx.x;
    const int total = tiles_m * tiles_n;
    if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
    const int grw = 4 * tiles_n, first = (t / grw) * 4, nrows = min(4, tiles_m - first);
    // (the tile indices are wave-uniform; saying so keeps the buffer
    // descriptors in scalar registers)
    const int tm = __builtin_amdgcn_readfirstlane(first + (t % grw) % nrows);
    const int tn = __builtin_amdgcn_readfirstlane((t % grw) / nrows);
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

    // the thread's share of a stage: 16-byte half gt % 2 of the stage's 32
    // code bytes of one tile row of A and of B, rows 128 grp .. 128 grp + 127.
    // Two lanes read a row's 32 bytes (16-byte pieces of separate rows load
    // at a quarter of the rate).  Each 16 lanes cover 8 rows, the even ones in
    // lanes 0-7 and the odd ones in lanes 8-15: rows 2j and 2j+1 share a
    // swizzle key, and 8 lanes that write one chunk of four rows of distinct
    // keys hit distinct banks (a probe: 13 cycles per 1 KiB written, as for
    // contiguous writes, against 16 with consecutive rows in lanes 0-7).
    const int crow = 128 * grp + (gt >> 4) * 8 + ((gt >> 1) & 3) * 2 + ((gt >> 3) & 1), chalf = gt & 1;
    const uint32_t co = (uint32_t)(crow * kcb) + (uint32_t)(chalf * 16);
    const uint32_t so = (uint32_t)(crow * ksb) + (uint32_t)(chalf * 2);
    // two register sets of loaded codes and scales, by stage parity: a
    // group's half of stage s+3 is loaded while it converts stage s+1, so
    // each load has two stages to arrive
    uint4 cA[2], cB[2];
    uint32_t sA[2], sB[2];
    auto gload = [&](auto PC, int s) __attribute__((always_inline)) {
        constexpr int P = decltype(PC)::value;
        cA[P] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rA, co, s * 32, 0));
        cB[P] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rB, co, s * 32, 0));
        sA[P] = __builtin_amdgcn_raw_buffer_load_b16(rSA, so, s * 4, 0);
        sB[P] = __builtin_amdgcn_raw_buffer_load_b16(rSB, so, s * 4, 0);
    };
    auto dq_write = [&](auto PC, int buf) __attribute__((always_inline)) {
        constexpr int P = decltype(PC)::value;
        // the row goes through an empty asm so that its LDS addresses are
        // formed here, in the conversion phase, rather than held in registers
        // across the loop
        int r = crow;
        asm volatile("" : "+v"(r));
        nv_dequant_chunk(tA(buf), r, chalf, cA[P], sA[P]);
        nv_dequant_chunk(tB(buf), r, chalf, cB[P], sB[P]);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    f16acc acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // stage 0 by both groups, then each group's halves of stages 1 and 2 in flight
    gload(P0{}, 0);
    dq_write(P0{}, 0);
    if (nst > 1) gload(P1{}, 1);
    if (nst > 2) gload(P0{}, 2);
    lds_barrier();
    // fragments of k-step ks of buffer `buf`: A tiles 0..3 and B tiles 0..1 of the wave
    struct Frag { h8 a[4], b[2]; };
    const int arow = wm * 128 + l32, brow = wn * 128 + grp * 64 + l32;
    auto rd_frags = [&](Frag& f, int buf, int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; i++) f.a[i] = *(const h8*)(tA(buf) + nv_swz(arow + i * 32, 2 * ks + h));
#pragma unroll
        for (int j = 0; j < 2; j++) f.b[j] = *(const h8*)(tB(buf) + nv_swz(brow + j * 32, 2 * ks + h));
    };
    auto mmas = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    // each k-step's fragments are read while the previous k-step's MFMAs
    // run (two register sets); the fences keep the reads ahead of the MFMAs
    Frag F0, F1;
    // stage s (parity P = s & 1): buffer P holds it; the converting group
    // writes its half of stage s+1 into buffer P^1 from register set P^1,
    // then loads its half of stage s+3 into that set
    auto stage = [&](auto PC, int s) __attribute__((always_inline)) {
        constexpr int P = decltype(PC)::value;
        using Q = std::integral_constant<int, P ^ 1>;
        for (int p = 0; p < 2; p++) {
            if (grp == p) {
                rd_frags(F0, P, 0);
                __builtin_amdgcn_sched_barrier(0);
                rd_frags(F1, P, 1);
                __builtin_amdgcn_sched_barrier(0);
                mmas(F0);
                __builtin_amdgcn_sched_barrier(0);
                rd_frags(F0, P, 2);
                __builtin_amdgcn_sched_barrier(0);
                mmas(F1);
                __builtin_amdgcn_sched_barrier(0);
                rd_frags(F1, P, 3);
                __builtin_amdgcn_sched_barrier(0);
                mmas(F0);
                __builtin_amdgcn_sched_barrier(0);
                mmas(F1);
                __builtin_amdgcn_sched_barrier(0);
            } else if (s + 1 < nst) {
                dq_write(Q{}, P ^ 1);                // this group's half of stage s+1
                if (s + 3 < nst) gload(Q{}, s + 3);
            }
            // LDS hand-off only: the loads stay in flight across it
            lds_barrier();
        }
    };
    for (int s = 0; s < nst; s += 2) {
        stage(P0{}, s);
        if (s + 1 < nst) stage(P1{}, s + 1);
    }

    // epilogue: alpha and the two second-level scales once per output
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + wn * 128 + grp * 64 + j * 32 + l32;
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
    const int64_t es = SRC == SRC_BF16 ? 2 : 4;
    const bool vec = ((uintptr_t)j.x % 16) == 0 && (j.ld * es) % 16 == 0 && j.cols % 8 == 0;
    // (source offsets within a panel stay below 2^31 bytes)
    if (SRC == SRC_BF16 && j.local && vec && L <= NV_FUSED_MAXL && (ROW ? 32 : L) * j.ld * es < ((int64_t)1 << 31)) {
        // CTA-local, one pass: the panel fits one workgroup's registers
        k_nv_quant_local<ROW><<<(unsigned)std::min<int64_t>(npanels, 65535), NV_FUSED_THREADS, 0, st>>>(
            (const uint16_t*)j.x, j.rows, j.cols, j.ld, npanels, j.ts, j.q, j.s16);
        return hipGetLastError();
    }
    // amax partials: about 2048 workgroups; parked in the code array, which
    // the quantize kernel overwrites afterwards (npanels * G * 4 bytes is at
    // most rows * cols / 4, the array holds rows * cols / 2)
    const int tiles_r = (int)((j.rows + 31) / 32), tiles_c = (int)((j.cols + 255) / 256);
    const int across = ROW ? tiles_r : tiles_c, along = ROW ? tiles_c : tiles_r;
    int G = (int)std::max<int64_t>(1, std::min<int64_t>(along, 2048 / std::max(1, across)));
    const int S = (along + G - 1) / G;
    G = (along + S - 1) / S;
    uint32_t* partial = (uint32_t*)j.q;
    const int64_t nwg = (int64_t)across * G;
    k_nv_amax<SRC, ROW><<<(unsigned)std::min<int64_t>(nwg, 65535), 256, 0, st>>>(j.x, j.rows, j.cols, j.ld, vec, across,
                                                                                  along, S, G, npanels, partial);
    if (j.local)
        k_nv_scales_local<<<(unsigned)((npanels + 255) / 256), 256, 0, st>>>(partial, npanels, G, j.ts);
    else
        k_nv_scale_global<<<1, 1024, 0, st>>>(partial, npanels * G, j.ts);
    if (ROW) {
        k_nv_quant_row<SRC><<<nv_grid(j.rows * (j.cols / 16)), 256, 0, st>>>(j.x, j.rows, j.cols, j.ld, vec, j.local,
                                                                            j.ts, j.q, j.s16);
    } else {
        const int64_t tiles = ((j.rows + 127) / 128) * ((j.cols + 63) / 64);
        k_nv_quant_col<SRC><<<(unsigned)std::min<int64_t>(tiles, 65535), 256, 0, st>>>(j.x, j.rows, j.cols, j.ld, vec,
                                                                                      j.local, j.ts, j.q, j.s16);
    }
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
    if (j.out_dtype == 0) k_nv_gemm<0><<<grid, 512, 0, stream>>>(j, tiles_m, tiles_n);
    else k_nv_gemm<1><<<grid, 512, 0, stream>>>(j, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace mx
