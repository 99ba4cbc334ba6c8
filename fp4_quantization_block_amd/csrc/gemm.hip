// gemm.hip -- block-scaled MX GEMM on gfx950 scaled MFMA.
//
// [MOSS, "GEMM Kernel 优化"]: the main loop is pure matrix-core work on the
// scaled codes -- here V_MFMA_SCALE_F32_32X32X64_F8F6F4 applies the E8M0
// block scales inside the instruction, so there is no dequantization in the
// K loop -- and the per-tensor FP32 scales (two-level scheme) are applied
// once, in the epilogue.
//
// Sources:
//   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
//
// C[M][N] = alpha' * A[M][K] . B[N][K]^T, A/B as written by the quantizer
// (K contiguous codes, [rows][K/32] E8M0 scales).
//
// Tiling: 256x256 output tile per 256-thread workgroup (2x2 waves, 128x128
// per wave = 4x4 MFMA 32x32 tiles with fp32 accumulators); K advances 128
// bytes per row per stage (128 FP8 / 256 FP4 elements); A and B stages are
// double-buffered in LDS (2 x 64 KiB + scales) with an XOR swizzle of the
// 16-byte chunks to keep ds_read_b128 conflict-free.
//
// Operand lane layout of the 32x32x64 scaled MFMA (lane l, h = l / 32, row
// or column l % 32):
//   FP8: bytes 0-15 hold K [16h, 16h+16), bytes 16-31 hold K [32+16h, ...);
//        the scale of K-block b (b = 0, 1) comes from lane (row + 32 b).
//   FP4: 16 bytes hold K [32h, 32h+32), element 2j in the low nibble of
//        byte j; the lane's own scale covers its block.
// Either way lane l supplies the scale byte of block (2*kstep + h) of its
// row, which is what the scale registers below carry.
// Accumulator layout: register r of lane l is C[8(r/4) + 4h + r%4][l%32].
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                  // bytes of K per row per stage
constexpr int TILE_BYTES = BM * BKB;      // 32 KiB per operand per stage
constexpr int SCALE_BYTES_MAX = 8;        // scale bytes per row per stage (FP4)

struct GArgs {
    const uint8_t* qa; const uint8_t* sa; const float* ta;
    const uint8_t* qb; const uint8_t* sb; const float* tb;
    int64_t M, N, K;
    float alpha; int hadamard_k;
    void* c; int64_t ldc;
    int tiles_m, tiles_n;
};

// MFMA format codes: 0 = E4M3, 1 = E5M2, 4 = E2M1
template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<E4M3> { static constexpr int code = 0; };
template <> struct MfmaFmt<E5M2> { static constexpr int code = 1; };
template <> struct MfmaFmt<E2M1> { static constexpr int code = 4; };

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm(GArgs g)
{
    constexpr bool FP4 = (FA == E2M1);
    constexpr int EPB = FP4 ? 2 : 1;                 // elements per byte
    constexpr int SB = BKB * EPB / 32;               // scale bytes per row per stage (4 or 8)
    constexpr int KSTEPS = BKB * EPB / 64;           // MFMA k-steps per stage (2 or 4)

    extern __shared__ __align__(16) uint8_t smem[];
    // stage buffers: [A0 B0 A1 B1] tiles, then [SA0 SB0 SA1 SB1] scales
    auto sA = [&](int buf) { return smem + buf * 2 * TILE_BYTES; };
    auto sB = [&](int buf) { return smem + buf * 2 * TILE_BYTES + TILE_BYTES; };
    auto sSA = [&](int buf) { return smem + 4 * TILE_BYTES + buf * 2 * BM * SCALE_BYTES_MAX; };
    auto sSB = [&](int buf) { return smem + 4 * TILE_BYTES + buf * 2 * BM * SCALE_BYTES_MAX + BM * SCALE_BYTES_MAX; };

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    // workgroup -> tile: consecutive ids run down a band of 8 tile rows so the
    // A rows and B columns a wave of workgroups touches stay in L2
    const int wg = blockIdx.x;
    const int band = 8;
    const int tiles_in_band = band * g.tiles_n;
    const int b_idx = wg / tiles_in_band;
    const int in_band = wg - b_idx * tiles_in_band;
    const int band_rows = min(band, g.tiles_m - b_idx * band);
    const int tm = b_idx * band + in_band % band_rows;
    const int tn = in_band / band_rows;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int64_t kbytes = g.K / EPB;                // bytes per operand row
    const int64_t kblocks = g.K / 32;
    const int nstages = (int)((kbytes + BKB - 1) / BKB);

    // ---- global -> register staging (8 chunks of 16 B per operand per thread) ----
    uint4 ra[8], rb[8];
    uint32_t rsa[SB / 4], rsb[SB / 4];

    auto load_stage = [&](int s) {
        const int64_t kb0 = (int64_t)s * BKB;
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int id = p * 256 + tid;
            const int row = id >> 3, chunk = id & 7;
            const int64_t kb = kb0 + chunk * 16;
            const int64_t ar = min(m0 + row, g.M - 1), br = min(n0 + row, g.N - 1);
            if (kb < kbytes) {
                ra[p] = *(const uint4*)(g.qa + ar * kbytes + kb);
                rb[p] = *(const uint4*)(g.qb + br * kbytes + kb);
            } else {
                ra[p] = make_uint4(0, 0, 0, 0);
                rb[p] = make_uint4(0, 0, 0, 0);
            }
        }
        // scales: one row per thread
        const int64_t blk0 = (int64_t)s * SB;
        const int64_t ar = min(m0 + tid, g.M - 1), br = min(n0 + tid, g.N - 1);
#pragma unroll
        for (int w = 0; w < SB / 4; w++) {
            uint32_t va = 0, vb = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int64_t blk = blk0 + w * 4 + b;
                const uint32_t xa = blk < kblocks ? g.sa[ar * kblocks + blk] : 127u;
                const uint32_t xb = blk < kblocks ? g.sb[br * kblocks + blk] : 127u;
                va |= xa << (8 * b);
                vb |= xb << (8 * b);
            }
            rsa[w] = va;
            rsb[w] = vb;
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int id = p * 256 + tid;
            const int row = id >> 3, chunk = id & 7;
            *(uint4*)(sA(buf) + swz(row, chunk)) = ra[p];
            *(uint4*)(sB(buf) + swz(row, chunk)) = rb[p];
        }
#pragma unroll
        for (int w = 0; w < SB / 4; w++) {
            ((uint32_t*)(sSA(buf) + tid * SCALE_BYTES_MAX))[w] = rsa[w];
            ((uint32_t*)(sSB(buf) + tid * SCALE_BYTES_MAX))[w] = rsb[w];
        }
    };

    f16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int s = 0; s < nstages; s++) {
        const int buf = s & 1;
        if (s + 1 < nstages) load_stage(s + 1);

        // scale registers: lane's row, shifted so block (2*ks + h) sits at byte 2*(ks%2)
        uint32_t sca[4][SB / 4], scb[4][SB / 4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ra_row = wm * 128 + i * 32 + l32;
            const int rb_row = wn * 128 + i * 32 + l32;
#pragma unroll
            for (int w = 0; w < SB / 4; w++) {
                sca[i][w] = ((const uint32_t*)(sSA(buf) + ra_row * SCALE_BYTES_MAX))[w] >> (8 * h);
                scb[i][w] = ((const uint32_t*)(sSB(buf) + rb_row * SCALE_BYTES_MAX))[w] >> (8 * h);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            int8v fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int ra_row = wm * 128 + i * 32 + l32;
                const int rb_row = wn * 128 + i * 32 + l32;
                if constexpr (!FP4) {
                    const uint4 a0 = *(const uint4*)(sA(buf) + swz(ra_row, ks * 4 + h));
                    const uint4 a1 = *(const uint4*)(sA(buf) + swz(ra_row, ks * 4 + 2 + h));
                    const uint4 b0 = *(const uint4*)(sB(buf) + swz(rb_row, ks * 4 + h));
                    const uint4 b1 = *(const uint4*)(sB(buf) + swz(rb_row, ks * 4 + 2 + h));
                    fa[i] = int8v{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                    fb[i] = int8v{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                } else {
                    const uint4 a0 = *(const uint4*)(sA(buf) + swz(ra_row, ks * 2 + h));
                    const uint4 b0 = *(const uint4*)(sB(buf) + swz(rb_row, ks * 2 + h));
                    fa[i] = int8v{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
                    fb[i] = int8v{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int w = ks / 2;                 // scale dword
                    if ((ks & 1) == 0)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[i], fb[j], acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code,
                            0, (int)sca[i][w], 0, (int)scb[j][w]);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fa[i], fb[j], acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code,
                            2, (int)sca[i][w], 2, (int)scb[j][w]);
                }
        }
        if (s + 1 < nstages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: per-tensor scales once ----
    float ap = g.alpha;
    if (g.ta) ap = ap * *g.ta;
    if (g.tb) ap = ap * *g.tb;
    if (g.hadamard_k) ap = ap * 0.03125f;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int64_t col = n0 + wn * 128 + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                if (row < g.M && col < g.N) {
                    const float v = acc[i][j][r] * ap;
                    if constexpr (OUT == 0) ((float*)g.c)[row * g.ldc + col] = v;
                    else ((uint16_t*)g.c)[row * g.ldc + col] = f32_to_bf16_rne(v);
                }
            }
        }
}

constexpr size_t kSmemBytes = 4 * TILE_BYTES + 4 * BM * SCALE_BYTES_MAX;   // 136 KiB

template <int FA, int FB, int OUT>
hipError_t launch3(const GArgs& a, hipStream_t s)
{
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_gemm<FA, FB, OUT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const unsigned nwg = (unsigned)(a.tiles_m * a.tiles_n);
    k_gemm<FA, FB, OUT><<<dim3(nwg), dim3(256), kSmemBytes, s>>>(a);
    return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch2(const GArgs& a, int out, hipStream_t s)
{
    return out == 0 ? launch3<FA, FB, 0>(a, s) : launch3<FA, FB, 1>(a, s);
}

}  // namespace

hipError_t launch_gemm(const GemmJob& j, hipStream_t stream)
{
    GArgs a;
    a.qa = j.qa; a.sa = j.sa; a.ta = j.ta;
    a.qb = j.qb; a.sb = j.sb; a.tb = j.tb;
    a.M = j.M; a.N = j.N; a.K = j.K;
    a.alpha = j.alpha; a.hadamard_k = j.hadamard_k;
    a.c = j.c; a.ldc = j.ldc;
    a.tiles_m = (int)((j.M + BM - 1) / BM);
    a.tiles_n = (int)((j.N + BN - 1) / BN);
    if (j.fa == E2M1) return launch2<E2M1, E2M1>(a, j.out_dtype, stream);
    if (j.fa == E4M3 && j.fb == E4M3) return launch2<E4M3, E4M3>(a, j.out_dtype, stream);
    if (j.fa == E5M2 && j.fb == E4M3) return launch2<E5M2, E4M3>(a, j.out_dtype, stream);
    if (j.fa == E4M3 && j.fb == E5M2) return launch2<E4M3, E5M2>(a, j.out_dtype, stream);
    return launch2<E5M2, E5M2>(a, j.out_dtype, stream);
}

}  // namespace mx
