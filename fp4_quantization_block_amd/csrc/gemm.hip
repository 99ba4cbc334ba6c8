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
//   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践"
//
// C[M][N] = alpha' * A[M][K] . B[N][K]^T, A/B as written by the quantizer
// (K contiguous codes, [rows][K/32] E8M0 scales).  The output is fp32,
// bf16, or -- [FAF, "格式感知融合的设计思路"], the producer writing its
// consumer's format -- FP8 codes with E8M0 1x32 row scales.
//
// Two kernels.  k_gemm_w4 (one wave per SIMD, described at its definition)
// runs every GEMM whose rows of K hold a multiple of 128 bytes of codes and
// whose scale arrays are 4-byte aligned, and is the only one with the
// MX-quantized output.  k_gemm below takes the rest (a ragged last K stage,
// unaligned scale arrays):
//
// Tiling: 256x256 output tile per 512-thread workgroup (2x4 waves, 128x64
// per wave = 4x2 MFMA 32x32 tiles, fp32 accumulators in AGPRs).  Two waves
// share each SIMD.  They run a two-group schedule: waves 0-3 and 4-7
// alternate phases one MFMA k-step long, one group issuing the MFMAs of a
// k-step from registers while the other reads its next operands from LDS,
// with a fence-free workgroup barrier between phases.  K advances 128 bytes
// per row per stage (128 FP8 / 256 FP4 elements).  Stages are double-buffered
// in LDS and filled by direct global->LDS loads (buffer_load_dwordx4 ... lds:
// lane i of a wave writes bytes [16i, 16i+16) of a 1 KiB run), so operand
// tiles never pass through VGPRs.  Waves 0-3 issue those loads, spread over
// their first read phase and first MFMA phase of a stage.  The per-CU rate
// of these loads (about 64 GB/s measured) is as much of a limit as the MFMA
// rate at this tile size: one stage's 64 KiB take about as long to arrive
// as the stage's MFMAs take to run.
// The 16-byte chunks of each 128-byte LDS row are XOR-swizzled by
// (row >> 1) & 7 -- applied on the global side by choosing which chunk each
// lane fetches -- which keeps the ds_read_b128 operand fetches free of bank
// conflicts.  A ragged last K stage (K not a multiple of the stage) is loaded
// through registers with zero fill.
//
// Operand lane layout of the 32x32x64 scaled MFMA (lane l, h = l / 32, row
// or column l % 32), established with on-device probes:
//   FP8: bytes 0-15 hold K [16h, 16h+16), bytes 16-31 hold K [32+16h, ...);
//        the scale of K-block b (b = 0, 1) comes from lane (row + 32 b).
//   FP4: 16 bytes hold K [32h, 32h+32), element 2j in the low nibble of
//        byte j; the lane's own scale covers its block.
// Either way lane l supplies the scale byte of block (2*kstep + h) of its
// row.  Accumulator register r of lane l is C[8(r/4) + 4h + r%4][l%32].
//
// Workgroup order: workgroups are dealt round-robin to the 8 XCDs (each
// with its own L2); the tile order below gives each XCD a compact block of
// tiles (4 tile rows x 8 tile columns when the grid allows), so the A rows
// and B columns one XCD streams are shared by its tiles through its L2.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256;
constexpr int BKB = 128;                  // bytes of K per row per stage
constexpr int TILE_BYTES = BM * BKB;      // 32 KiB per operand per stage
constexpr int GROUP_M = 4;                // tile rows per ordering group

struct GArgs {
    const uint8_t* qa; const uint8_t* sa; const float* ta;
    const uint8_t* qb; const uint8_t* sb; const float* tb;
    int64_t M, N, K;
    float alpha; int hadamard_k;
    void* c; int64_t ldc;
    uint8_t* cs;              // MX-quantized output: [M][N/32] scale bytes (c holds [M][N] codes)
    int tiles_m, tiles_n;
    int reg_path;             // 1: scale arrays not 4-byte aligned -> every stage via registers
};

template <int FMT> struct MfmaFmt;
template <> struct MfmaFmt<E4M3> { static constexpr int code = 0; };
template <> struct MfmaFmt<E5M2> { static constexpr int code = 1; };
template <> struct MfmaFmt<E2M1> { static constexpr int code = 4; };

// LDS byte offset of 16-byte chunk `chunk` of tile row `row`.  The XOR key (row >> 1) & 7
// together with the row parity spreads 16 consecutive rows over all 64 banks,
// so the 16 lanes a ds_read_b128 serves per cycle never collide.
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ swz_key(row)) << 4); }

// Two fp32 values to bf16 with round-to-nearest-even in one packed convert.
// The epilogue runs once per tile as straight-line code that is fetched
// cold on every launch; one convert per pair instead of a five-instruction
// software rounding per value halves that code (and measurably the
// kernel's fixed cost).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// tile index of this workgroup: XCD-aware, then grouped row-major order
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    int t = wg;
    if (total % 8 == 0) {                     // workgroup wg runs on XCD wg % 8
        const int per = total / 8;
        t = (wg % 8) * per + wg / 8;
    }
    const int group = GROUP_M * tiles_n;
    const int g = t / group;
    const int first = g * GROUP_M;
    const int rows = min(GROUP_M, tiles_m - first);
    const int in = t - g * group;
    tm = first + in % rows;
    tn = in / rows;
}

// Ties the accumulators to this point of the program: the MFMA builtins
// have no side effects, so without it the compiler may sink a phase's MFMAs
// past the barrier that ends the phase.
__device__ __forceinline__ void pin(f16v (&acc)[4][2])
{
#if defined(__HIP_DEVICE_COMPILE__)      // AGPR constraint: device pass only
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) asm volatile("" : "+a"(acc[i][j]));
#endif
}

// Operands of one MFMA k-step (64 elements of K) for a wave's 128x64
// sub-tile, held in registers from the read phase to the MFMA phase of the
// two-group schedule; scale dwords pre-shifted so the lane's block sits at
// byte 2*(ks%2).
// (FP4 operands fill only the low half of the MFMA's 8-dword source: the
// instruction reads 4 registers for that format, so only those are held.)
typedef int int4v __attribute__((ext_vector_type(4)));
template <bool FP4>
struct KFrag {
    typedef typename std::conditional<FP4, int4v, int8v>::type V;
    V a[4], b[2];
    uint32_t sa[4], sb[2];
};

template <bool FP4>
__device__ __forceinline__ int8v mfma_src(const typename KFrag<FP4>::V& v)
{
    if constexpr (FP4) return int8v{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    else return v;
}

// Lane offsets into an operand tile, re-derived in every read phase: they
// pass through an empty asm first, so the compiler recomputes the few
// addresses of a phase from them instead of keeping every phase's addresses
// live across the whole K loop.
struct LaneOffs {
    uint32_t a, b;        // byte offset of the lane's first A / B row (row * BKB)
    uint32_t hk;          // (h ^ swizzle key of the lane's rows) << 4
    uint32_t sa, sb;      // scale-plane index of the lane's first A / B row
};

template <bool FP4>
__device__ __forceinline__ void read_kstep(KFrag<FP4>& f, const uint8_t* sA, const uint8_t* sB,
                                           const uint32_t* sSA, const uint32_t* sSB, int ks, LaneOffs o,
                                           int h)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(o.a), "+v"(o.b), "+v"(o.hk), "+v"(o.sa), "+v"(o.sb));
#endif
    // chunk (c ^ key) of the lane's rows, for c = cbase + h: rows 32 apart
    // share the key, so one offset serves all row tiles of the operand
    auto cofs = [&](int cbase) { return ((uint32_t)cbase << 4) ^ o.hk; };
    auto frag = [&](const uint8_t* base, uint32_t lane_off, int t) {
        if constexpr (!FP4) {
            const uint4 c0 = *(const uint4*)(base + lane_off + cofs(ks * 4) + t * 32 * BKB);
            const uint4 c1 = *(const uint4*)(base + lane_off + cofs(ks * 4 + 2) + t * 32 * BKB);
            return int8v{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w, (int)c1.x, (int)c1.y, (int)c1.z, (int)c1.w};
        } else {
            const uint4 c0 = *(const uint4*)(base + lane_off + cofs(ks * 2) + t * 32 * BKB);
            return int4v{(int)c0.x, (int)c0.y, (int)c0.z, (int)c0.w};
        }
    };
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f.a[i] = frag(sA, o.a, i);
        f.sa[i] = sSA[(ks / 2) * BM + o.sa + i * 32] >> (8 * h);
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        f.b[j] = frag(sB, o.b, j);
        f.sb[j] = sSB[(ks / 2) * BM + o.sb + j * 32] >> (8 * h);
    }
}

// Makes the operands look redefined at this point of the program, so that
// the MFMAs that use them cannot be hoisted above it (they have no memory
// side effects, and the phase barriers only order memory).
template <bool FP4>
__device__ __forceinline__ void hold(KFrag<FP4>& f)
{
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0]), "+v"(f.b[1]));
    asm volatile("" : "+v"(f.sa[0]), "+v"(f.sa[1]), "+v"(f.sa[2]), "+v"(f.sa[3]), "+v"(f.sb[0]), "+v"(f.sb[1]));
#endif
}

// One k-step of MFMAs; after MFMA m (0..7) calls between(m), in program order.
template <int FA, int FB, typename Between>
__device__ __forceinline__ void mma_kstep_with(f16v (&acc)[4][2], const KFrag<FA == E2M1>& f, int ks, Between between)
{
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            if ((ks & 1) == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mfma_src<FA == E2M1>(f.a[i]), mfma_src<FA == E2M1>(f.b[j]), acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code, 0, (int)f.sa[i], 0,
                    (int)f.sb[j]);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mfma_src<FA == E2M1>(f.a[i]), mfma_src<FA == E2M1>(f.b[j]), acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code, 2, (int)f.sa[i], 2,
                    (int)f.sb[j]);
            __builtin_amdgcn_sched_barrier(0);
            between(2 * i + j);
            __builtin_amdgcn_sched_barrier(0);
        }
}

template <int FA, int FB>
__device__ __forceinline__ void mma_kstep(f16v (&acc)[4][2], const KFrag<FA == E2M1>& f, int ks)
{
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            if ((ks & 1) == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mfma_src<FA == E2M1>(f.a[i]), mfma_src<FA == E2M1>(f.b[j]), acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code, 0, (int)f.sa[i], 0,
                    (int)f.sb[j]);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    mfma_src<FA == E2M1>(f.a[i]), mfma_src<FA == E2M1>(f.b[j]), acc[i][j], MfmaFmt<FA>::code, MfmaFmt<FB>::code, 2, (int)f.sa[i], 2,
                    (int)f.sb[j]);
        }
}

// Workgroup barrier between the phases of the two-group schedule: this wave's LDS reads complete, no
// vector-memory wait, and the memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void half_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int FA, int FB, int OUT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm(GArgs g)
{
#if defined(__HIP_DEVICE_COMPILE__)      // the host pass only needs the launch stub
    constexpr bool FP4 = (FA == E2M1);
    constexpr int EPB = FP4 ? 2 : 1;                 // elements per byte
    constexpr int SB = BKB * EPB / 32;               // scale bytes per row per stage (4 or 8)
    constexpr int KSTEPS = BKB * EPB / 64;           // MFMA k-steps per stage (2 or 4)

    // Two stage buffers as distinct LDS objects: the compiler can then see
    // that fragment reads of one buffer do not depend on the direct loads
    // still filling the other, and does not wait for them.
    __shared__ __align__(16) uint8_t lA0[TILE_BYTES], lA1[TILE_BYTES];
    __shared__ __align__(16) uint8_t lB0[TILE_BYTES], lB1[TILE_BYTES];
    __shared__ __align__(16) uint32_t lSA0[2 * BM], lSA1[2 * BM], lSB0[2 * BM], lSB1[2 * BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
    const int wm = wave >> 2, wn = wave & 3;
    const int h = lane >> 5, l32 = lane & 31;

    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int64_t kbytes = g.K / EPB;                // bytes per operand row
    const int64_t kblocks = g.K / 32;
    const int nstages = (int)((kbytes + BKB - 1) / BKB);
    const bool ragged = (kbytes % BKB) != 0;

    // ---- stage loads ----
    // Loads are issued by waves 0-3 only.
    // direct: bounds-checked buffer loads straight into LDS.  Wave w, load p
    // covers tile rows 32p + 8w .. +8; lane -> row (lane / 8) of that run and
    // LDS slot (lane % 8), which receives global chunk slot ^ key(row).  The
    // buffer of a stage starts at tile row 0 and ends at row M (N), so rows
    // past the matrix read as zero.  Only the lane's 32-bit offset lives in a
    // VGPR.  Scales: wave w loads rows 64w .. +64 of both operands.
    const int lrow = 8 * (wave & 3) + (lane >> 3);            // row within a 32-row run
    const uint32_t voff = (uint32_t)(lrow * kbytes + (((lane & 7) ^ swz_key(lrow)) << 4));
    const uint32_t soff_row = (uint32_t)((64 * (wave & 3) + lane) * kblocks);
    // One descriptor per operand for the whole K loop, based at the tile's
    // first row and ending at row M (N); the stage's K offset is added to the
    // lane offset, so rows past the matrix still fall outside the range.
    auto rsrc = [&](const uint8_t* base, int64_t first_row, int64_t rows, int64_t row_bytes) __attribute__((always_inline)) {
        int64_t n = (rows - first_row) * row_bytes;
        n = n < 0 ? 0 : n > 0xFFFFFFFFll ? 0xFFFFFFFFll : n;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + first_row * row_bytes), (short)0,
                                                 (int)(uint32_t)n, 0x00020000);
    };
    const auto ra = rsrc(g.qa, m0, g.M, kbytes), rb = rsrc(g.qb, n0, g.N, kbytes);
    const auto rsa = rsrc(g.sa, m0, g.M, kblocks), rsb = rsrc(g.sb, n0, g.N, kblocks);
    // Operand load instruction q (0..15) of stage s: run p = q / 2 of A (q
    // even) or B (q odd); then the scale loads.
    auto dma_op = [&](int s, int q, uint8_t* sA, uint8_t* sB) __attribute__((always_inline)) {
        const int p = q >> 1;
        uint32_t v = voff;
#if defined(__HIP_DEVICE_COMPILE__)
        asm volatile("" : "+v"(v));
#endif
        const uint32_t off = v + (uint32_t)(s * BKB) + (uint32_t)(32 * p * kbytes);
        if (q & 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sB + (32 * p + 8 * wave) * BKB), 16, off, 0, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sA + (32 * p + 8 * wave) * BKB), 16, off, 0, 0, 0);
    };
    // scales: plane w holds bytes [4w, 4w+4) of every row's stage scales
    auto dma_scales = [&](int s, uint32_t* sSA, uint32_t* sSB) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < SB / 4; w++) {
            const uint32_t off = soff_row + (uint32_t)(s * SB + 4 * w);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(sSA + w * BM + 64 * wave), 4, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(sSB + w * BM + 64 * wave), 4, off, 0, 0, 0);
        }
    };
    auto load_direct = [&](int s, uint8_t* sA, uint8_t* sB, uint32_t* sSA, uint32_t* sSB) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 16; q++) dma_op(s, q, sA, sB);
        dma_scales(s, sSA, sSB);
    };
    // register path with zero fill for a ragged last stage
    auto load_tail = [&](int s, uint8_t* sA, uint8_t* sB, uint32_t* sSA, uint32_t* sSB) __attribute__((always_inline)) {
        const int64_t kb0 = (int64_t)s * BKB;
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int id = p * 256 + tid;
            const int row = id >> 3, chunk = id & 7;
            const int64_t kb = kb0 + chunk * 16;
            const int64_t ar = min(m0 + row, g.M - 1), br = min(n0 + row, g.N - 1);
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (kb < kbytes) {
                va = *(const uint4*)(g.qa + ar * kbytes + kb);
                vb = *(const uint4*)(g.qb + br * kbytes + kb);
            }
            *(uint4*)(sA + swz(row, chunk)) = va;
            *(uint4*)(sB + swz(row, chunk)) = vb;
        }
        const int64_t ar = min(m0 + tid, g.M - 1), br = min(n0 + tid, g.N - 1);
#pragma unroll
        for (int w = 0; w < SB / 4; w++) {
            uint32_t va = 0, vb = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int64_t blk = (int64_t)s * SB + 4 * w + b;
                const uint32_t xa = blk < kblocks ? g.sa[ar * kblocks + blk] : 127u;
                const uint32_t xb = blk < kblocks ? g.sb[br * kblocks + blk] : 127u;
                va |= xa << (8 * b);
                vb |= xb << (8 * b);
            }
            sSA[w * BM + tid] = va;
            sSB[w * BM + tid] = vb;
        }
    };
    auto load_stage = [&](int s, uint8_t* sA, uint8_t* sB, uint32_t* sSA, uint32_t* sSB) __attribute__((always_inline)) {
        if (g.reg_path || (ragged && s == nstages - 1)) load_tail(s, sA, sB, sSA, sSB);
        else load_direct(s, sA, sB, sSA, sSB);
    };

    f16v acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // Two-group schedule.  Waves 0-3 (group 0: rows 0-127 of the tile) and
    // waves 4-7 (group 1: rows 128-255) share the SIMDs pairwise and
    // alternate phases one MFMA k-step long: while one group runs the MFMAs
    // of a k-step from registers, the other reads its operands of the next
    // k-step from LDS, so each SIMD always holds a wave whose operands are
    // ready.  With t counting k-steps over the whole K loop:
    //   phase 2t-1: group 0 reads k-step t       | group 1 MFMAs of t-1
    //   phase 2t  : group 0 MFMAs of k-step t    | group 1 reads t
    // Group 0 also drives the loads: stage s+1 is issued in the phase where
    // group 0 reads the first k-step of stage s -- its buffer was last read
    // by group 1 in the phase before -- and awaited at the end of group 0's
    // MFMAs of the last k-step of stage s.  Every phase ends with a workgroup
    // barrier without a memory fence; both groups pass 2T+2 of them.
    LaneOffs lo;
    lo.a = (uint32_t)((wm * 128 + l32) * BKB);
    lo.b = (uint32_t)((wn * 64 + l32) * BKB);
    lo.hk = (uint32_t)((h ^ swz_key(l32)) << 4);
    lo.sa = (uint32_t)(wm * 128 + l32);
    lo.sb = (uint32_t)(wn * 64 + l32);
    KFrag<FP4> f;
    // FAST: every load is direct (no register path, no ragged stage); the
    // other case keeps its loads out of the MFMA phases.
    auto g0_stage = [&](auto fast, int s, const uint8_t* xA, const uint8_t* xB, const uint32_t* xSA,
                        const uint32_t* xSB, uint8_t* yA, uint8_t* yB, uint32_t* ySA,
                        uint32_t* ySB) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast)::value;
        // In the fast case the next stage's loads are spread over the first
        // read phase (scales and the first half) and the MFMAs of the first
        // k-step (one instruction after each MFMA), so that no phase waits
        // for the address unit to take all of them at once.
        const bool next = s + 1 < nstages;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            read_kstep<FP4>(f, xA, xB, xSA, xSB, ks, lo, h);
            if (ks == 0 && next) {
                if constexpr (FAST) {
                    dma_scales(s + 1, ySA, ySB);
#pragma unroll
                    for (int q = 0; q < 8; q++) dma_op(s + 1, q, yA, yB);
                } else {
                    load_stage(s + 1, yA, yB, ySA, ySB);
                }
            }
            half_barrier();
            hold(f);
            if (FAST && ks == 0 && next)
                mma_kstep_with<FA, FB>(acc, f, ks, [&](int m) __attribute__((always_inline)) { dma_op(s + 1, 8 + m, yA, yB); });
            else
                mma_kstep<FA, FB>(acc, f, ks);
            pin(acc);
            __builtin_amdgcn_sched_barrier(0);
            if (ks == KSTEPS - 1) __builtin_amdgcn_s_waitcnt(0);
            half_barrier();
        }
    };
    auto g0_run = [&](auto fast) __attribute__((always_inline)) {
        if constexpr (decltype(fast)::value) load_direct(0, lA0, lB0, lSA0, lSB0);
        else load_stage(0, lA0, lB0, lSA0, lSB0);
        __builtin_amdgcn_s_waitcnt(0);
        half_barrier();                                        // stage 0 landed
        int s = 0;
        for (; s + 1 < nstages; s += 2) {
            g0_stage(fast, s, lA0, lB0, lSA0, lSB0, lA1, lB1, lSA1, lSB1);
            g0_stage(fast, s + 1, lA1, lB1, lSA1, lSB1, lA0, lB0, lSA0, lSB0);
        }
        if (s < nstages) g0_stage(fast, s, lA0, lB0, lSA0, lSB0, lA1, lB1, lSA1, lSB1);
        half_barrier();                                        // group 1's last MFMAs
    };
    auto g1_stage = [&](const uint8_t* xA, const uint8_t* xB, const uint32_t* xSA, const uint32_t* xSB) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            read_kstep<FP4>(f, xA, xB, xSA, xSB, ks, lo, h);
            half_barrier();
            hold(f);
            mma_kstep<FA, FB>(acc, f, ks);
            pin(acc);
            __builtin_amdgcn_sched_barrier(0);
            half_barrier();
        }
    };
    if (wave < 4) {
        if (g.reg_path || ragged) g0_run(std::false_type{});
        else g0_run(std::true_type{});
    } else {
        half_barrier();                                        // stage 0 landed
        half_barrier();                                        // group 0 reads k-step 0
        int s = 0;
        for (; s + 1 < nstages; s += 2) {
            g1_stage(lA0, lB0, lSA0, lSB0);
            g1_stage(lA1, lB1, lSA1, lSB1);
        }
        if (s < nstages) g1_stage(lA0, lB0, lSA0, lSB0);
    }

    // ---- epilogue: per-tensor scales once ----
    float ap = g.alpha;
    if (g.ta) ap = ap * *g.ta;
    if (g.tb) ap = ap * *g.tb;
    if (g.hadamard_k) ap = ap * 0.03125f;

    if constexpr (OUT == 1) {
        // bf16: each wave stages its 128x64 sub-tile (128-byte rows) in its
        // own 16 KiB of LDS, then writes 16-byte runs of 8 columns
        uint8_t* buf = (wave >> 1) == 0 ? lA0 : (wave >> 1) == 1 ? lA1 : (wave >> 1) == 2 ? lB0 : lB1;
        uint16_t* ct = (uint16_t*)(buf + (wave & 1) * 16384);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {     // rows r and r + 1 of the accumulator
                    const int row = i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    const int col = j * 32 + l32;
                    const uint32_t u = f32x2_to_bf16x2_rne(acc[i][j][r] * ap, acc[i][j][r + 1] * ap);
                    ct[row * 64 + col] = (uint16_t)u;
                    ct[(row + 1) * 64 + col] = (uint16_t)(u >> 16);
                }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const bool vec = (g.ldc % 8) == 0 && (((uintptr_t)g.c) & 15u) == 0;
        const int64_t rbase = m0 + wm * 128, cbase = n0 + wn * 64;
#pragma unroll 4
        for (int p = 0; p < 16; p++) {
            const int id = p * 64 + lane;
            const int row = id >> 3, c8 = (id & 7) * 8;
            const int64_t grow = rbase + row, gcol = cbase + c8;
            if (grow >= g.M) continue;
            const uint4 v = *(const uint4*)(ct + row * 64 + c8);
            uint16_t* dst = (uint16_t*)g.c + grow * g.ldc + gcol;
            if (vec && gcol + 8 <= g.N) {
                *(uint4*)dst = v;
            } else {
                const uint16_t* e = (const uint16_t*)&v;
                for (int k = 0; k < 8; k++)
                    if (gcol + k < g.N) dst[k] = e[k];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int64_t col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (row < g.M && col < g.N) ((float*)g.c)[row * g.ldc + col] = acc[i][j][r] * ap;
                }
            }
    }
#endif
}

// ---------------------------------------------------------------------------
// k_gemm_w4: rows of K holding a multiple of 128 bytes of codes (FP8: K %
// 128 == 0, FP4: K % 256 == 0) and 4-byte aligned scale arrays.  One wave
// per SIMD: a 256-thread workgroup computes a 256x256 tile, each wave a
// 128x128 quarter (4x4 MFMA 32x32 tiles, all 256 accumulator registers).
// Compared with two 128x64 waves per SIMD this reads a third less from LDS
// per MFMA (8 fragments per 16 MFMAs instead of 6 per 8), and lets each
// wave overlap its own loads with its MFMAs instead of trading phases with
// a partner wave at barriers.
//
// Operand tiles travel global -> registers -> LDS: each thread holds one
// stage's share (16 chunks of 16 bytes, 64 VGPRs) between its global load
// and its LDS write, which gives every load a whole stage to arrive.  A
// stage is 128 bytes of K per row: two MFMA k-steps for FP8, four for FP4.
// Each k-step is a phase of 16 MFMAs, each followed by one slot of other
// work: the LDS reads of the next k-step's fragments (the two fragment
// sets alternate), and the LDS writes and reloads of later stages.  One
// barrier per stage, before the last phase, which reads the next stage.
// LDS holds two stage buffers (2 x 64 KiB plus scales); the schedule of
// the writes into them is given at the main loop.  Rows past M (N) read as
// zero and their outputs are dropped; loads of stages past the end re-read
// the last stage into buffers nothing reads any more.
//
// Measured bound: with the loads taken out of the loop the same schedule
// runs the MFMAs at 77% of the FP8 peak at long K, so the loads set the
// pace.  Counters show each CU's vector-memory path saturated (address
// unit busy 65-93%, L1 waiting on pending L2 data 30-50% of cycles) at
// about 19 bytes per clock against the 32 a 256x256 FP8 tile needs at the
// MFMA rate, with an average L2 latency of 270-370 cycles.
// One 1x32 block of fp32 outputs to FP8 codes (FMT E4M3 / E5M2) and its
// E8M0 scale byte, the same encoding as the quantizer's row copies with
// round-to-nearest-even: shared exponent floor(log2 amax) - emax, exact
// scaling, saturation, and a NaN block (0x7F codes, byte 0xFF) when the
// block holds a NaN or Inf.
template <int FMT>
__device__ __forceinline__ uint32_t encode_out_block(const float (&v)[32], uint32_t* out)
{
    uint32_t key = 0;
#pragma unroll
    for (int k = 0; k < 32; k++) key = max(key, abs_key(v[k]));
    if (key >= 0x7F800000u) {
#pragma unroll
        for (int k = 0; k < 8; k++) out[k] = 0x7F7F7F7Fu;
        return 0xFFu;
    }
    const int e = block_exponent<FMT>(key);
#pragma unroll
    for (int k = 0; k < 8; k++)
        out[k] = cvt4_fp8<FMT>(clamp_fmax<FMT>(scale_by(v[4 * k], e)), clamp_fmax<FMT>(scale_by(v[4 * k + 1], e)),
                               clamp_fmax<FMT>(scale_by(v[4 * k + 2], e)), clamp_fmax<FMT>(scale_by(v[4 * k + 3], e)));
    return (uint32_t)(e + 127);
}

// k_gemm_w4's accumulators pinned to AGPRs (see pin above)
template <int JT>
__device__ __forceinline__ void pin4(f16v (&acc)[4][JT])
{
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < JT; j++) asm volatile("" : "+a"(acc[i][j]));
#endif
}

template <bool FP4, int JT>
struct W4Frag {
    typename KFrag<FP4>::V a[4], b[JT];
    uint32_t sa[4], sb[JT];
};

// Non-temporal stores for k_gemm_w4's output: nothing in the kernel reads C
// back, and streaming it past L2 measured 7-8% faster for the whole GEMM at
// 4096^3 and 8192x28672x4096 (the stores come in one burst at the end of
// every tile, with the matrix cores idle).  Single scale bytes stay cached:
// stored non-temporally they raised the bytes written by 30%.
__device__ __forceinline__ void store_nt16(void* p, uint4 v)
{
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, (u32x4v*)p);
}

// NB: tile columns (256, or 128 for the half tiles of a last partial round:
// each wave then computes 128 x 64 and the B tile has 128 rows).
template <int FA, int FB, int OUT, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_w4(GArgs g)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr bool FP4 = (FA == E2M1);
    constexpr int EPB = FP4 ? 2 : 1;                 // elements per byte
    constexpr int KS = BKB * EPB / 64;               // MFMA k-steps per stage (2 FP8, 4 FP4)
    constexpr int SBD = KS / 2;                      // scale dwords per row per stage
    constexpr int JT = NB / 64;                      // 32-column MFMA tiles per wave (4 or 2)
    constexpr int RB = NB / 32;                      // 32-row load runs of the B tile (8 or 4)
    constexpr int NM = 4 * JT;                       // MFMAs per k-step and wave
    static_assert(NB == 256 || (NB == 128 && OUT < 2), "half tiles serve the fp32 / bf16 outputs");
    typedef W4Frag<FP4, JT> Frag;
    __shared__ __align__(16) uint8_t lA0[TILE_BYTES], lA1[TILE_BYTES];
    __shared__ __align__(16) uint8_t lB0[NB * BKB], lB1[NB * BKB];
    // scale dwords of a stage, [A rows | B rows], in two planes: plane 1 holds
    // each dword shifted right by one byte, so a lane with h = 1 finds its
    // blocks at bytes 0 and 2 without a shift after the read
    // (SBD dwords per row per stage: [plane][dword][A rows | B rows])
    __shared__ __align__(16) uint32_t lS0[2 * SBD * 2 * BM], lS1[2 * SBD * 2 * BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;

    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * NB;
    const int64_t kbytes = g.K / EPB;
    const int64_t kblocks = g.K / 32;
    const int nstages = (int)(kbytes / BKB);

    // global loads of a stage: thread t moves 16-byte chunk (t & 7) of tile
    // rows 32p + t/8 (p = 0..7) of A and of B, and the stage's scale dword
    // of row t of A and of B.  Buffer loads: the row part of the offset is in
    // the range-checked lane offset, so rows past M (N) read as zero; the
    // stage's K offset rides in the unchecked scalar offset.
    auto rsrc = [&](const uint8_t* base, int64_t first_row, int64_t rows, int64_t row_bytes) __attribute__((always_inline)) {
        int64_t n = (rows - first_row) * row_bytes;
        n = n < 0 ? 0 : n > 0xFFFFFFFFll ? 0xFFFFFFFFll : n;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + first_row * row_bytes), (short)0,
                                                 (int)(uint32_t)n, 0x00020000);
    };
    // B rows past the tile (a half tile's other half) also read as zero
    const int64_t nend = min(g.N, n0 + NB);
    const auto ra = rsrc(g.qa, m0, g.M, kbytes), rb = rsrc(g.qb, n0, nend, kbytes);
    const auto rsa_ = rsrc(g.sa, m0, g.M, kblocks), rsb_ = rsrc(g.sb, n0, nend, kblocks);
    const int lr = tid >> 3, lc = tid & 7;
    const uint32_t voff = (uint32_t)(lr * kbytes + lc * 16);
    const uint32_t vsoff = (uint32_t)(tid * kblocks);
    const uint32_t prow = (uint32_t)(32 * kbytes);        // offset of run p: p * prow
    // LDS byte offset of the thread's chunk in run p: p * 32 * BKB + wofs
    const uint32_t wofs = (uint32_t)swz(lr, lc);

    uint4 stA[8], stB[RB];
    uint32_t stSA[SBD], stSB[SBD];
    // L2 warm-up: four stages ahead of its loads, each workgroup touches a
    // share of its A and B rows chosen so that the tiles sharing a panel on
    // one XCD (a block of 4 tile rows x 8 tile columns) touch different
    // rows -- 32 A rows by tile column, 64 B rows by tile row -- so most of
    // the panel is in L2 by the time its owners load it.  The loads go
    // straight to a scratch area of LDS that nothing reads (no registers).
    // Measured: the per-CU load path is bound by L2 latency, and misses to
    // the fabric are what raise it.
    __shared__ __align__(16) uint8_t lPF[4 * 1024];
    const uint32_t pfa = (uint32_t)((32 * (tn & 7) + 8 * wave + (lane >> 3)) * kbytes + (lane & 7) * 16);
    // (half tiles: 32 B rows by tile row, one load)
    const uint32_t pfb = (uint32_t)(((NB / 4) * (tm & 3) + (NB / 16) * wave + (lane >> 3)) * kbytes + (lane & 7) * 16);
    auto prefetch = [&](int s) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(lPF + wave * 1024), 16, pfa, s * BKB, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(lPF + wave * 1024), 16, pfb, s * BKB, 0, 0);
        if constexpr (NB == 256)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(lPF + wave * 1024), 16, pfb + 8 * (uint32_t)kbytes, s * BKB, 0, 0);
    };
    auto gl16 = [&](__amdgpu_buffer_rsrc_t r, int p, int s) __attribute__((always_inline)) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + p * prow, s * BKB, 0));
    };
    auto gload_scales = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < SBD; d++) {
            stSA[d] = __builtin_amdgcn_raw_buffer_load_b32(rsa_, vsoff, s * 4 * SBD + 4 * d, 0);
            stSB[d] = __builtin_amdgcn_raw_buffer_load_b32(rsb_, vsoff, s * 4 * SBD + 4 * d, 0);
        }
    };
    auto gload = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            stA[p] = gl16(ra, p, s);
            if (p < RB) stB[p] = gl16(rb, p, s);
        }
        gload_scales(s);
    };

    // fragment reads (same lane layout and swizzle as k_gemm)
    const uint32_t oa = (uint32_t)((wm * 128 + l32) * BKB);
    const uint32_t ob = (uint32_t)((wn * (NB / 2) + l32) * BKB);
    const uint32_t hk = (uint32_t)((h ^ swz_key(l32)) << 4);
    const int rsa = 2 * BM * SBD * h + wm * 128 + l32, rsb = 2 * BM * SBD * h + BM + wn * (NB / 2) + l32;
    // fragment t (0..3: A tile t, 4..7: B tile t-4) of k-step ks: FP8 holds
    // chunks 4ks + h and 4ks + 2 + h of the lane's row, FP4 chunk 2ks + h
    auto rd_frag = [&](Frag& f, const uint8_t* sA, const uint8_t* sB, int ks, int t) __attribute__((always_inline)) {
        const uint8_t* base = t < 4 ? sA + oa + (t & 3) * 32 * BKB : sB + ob + (t & 3) * 32 * BKB;
        typename KFrag<FP4>::V v;
        if constexpr (FP4) {
            const uint4 v0 = *(const uint4*)(base + ((((uint32_t)(ks * 2)) << 4) ^ hk));
            v = int4v{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w};
        } else {
            const uint4 v0 = *(const uint4*)(base + ((((uint32_t)(ks * 4)) << 4) ^ hk));
            const uint4 v1 = *(const uint4*)(base + ((((uint32_t)(ks * 4 + 2)) << 4) ^ hk));
            v = int8v{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
        if (t < 4) f.a[t] = v;
        else f.b[t - 4] = v;
    };
    // scale dword of tile t (t < 4: A, else B) for k-step ks: dword ks / 2
    // of the stage, with the lane's block at byte 2 * (ks % 2)
    auto rd_scale = [&](Frag& f, const uint32_t* sS, int t, int ks) __attribute__((always_inline)) {
        const int d = (ks / 2) * 2 * BM;
        if (t < 4) f.sa[t] = sS[d + rsa + 32 * t];
        else f.sb[t - 4] = sS[d + rsb + 32 * (t - 4)];
    };
    auto wr_scales = [&](uint32_t* sS) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < SBD; d++) {
            sS[d * 2 * BM + tid] = stSA[d];
            sS[d * 2 * BM + BM + tid] = stSB[d];
            sS[(SBD + d) * 2 * BM + tid] = stSA[d] >> 8;
            sS[(SBD + d) * 2 * BM + BM + tid] = stSB[d] >> 8;
        }
    };
    auto swrite_a = [&](uint8_t* sA, int p) __attribute__((always_inline)) { *(uint4*)(sA + p * 32 * BKB + wofs) = stA[p]; };
    auto swrite_b = [&](uint8_t* sB, int p) __attribute__((always_inline)) { *(uint4*)(sB + p * 32 * BKB + wofs) = stB[p]; };

    f16v acc[4][JT];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < JT; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    auto mma = [&](const Frag& f, int ks, int m) __attribute__((always_inline)) {
        const int i = m / JT, j = m % JT;
        if ((ks & 1) == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mfma_src<FP4>(f.a[i]), mfma_src<FP4>(f.b[j]), acc[i][j],
                                                                        MfmaFmt<FA>::code, MfmaFmt<FB>::code, 0, (int)f.sa[i], 0, (int)f.sb[j]);
        else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mfma_src<FP4>(f.a[i]), mfma_src<FP4>(f.b[j]), acc[i][j],
                                                                        MfmaFmt<FA>::code, MfmaFmt<FB>::code, 2, (int)f.sa[i], 2, (int)f.sb[j]);
    };

    pin4(acc);
    Frag F0, F1;
    // prologue: stage 0 into buffer 0 and stage 1's A tile into buffer 1;
    // stage 1's B tile and scales, and stage 2's A tile, left in flight
    // (stage 1 is loaded into temporaries before stage 0 is waited for, so
    // the two round trips overlap; the fragment registers are not live yet)
    {
        const int s1 = min(1, nstages - 1);
        gload(0);
        uint4 uA[8], uB[RB];
#pragma unroll
        for (int p = 0; p < 8; p++) {
            uA[p] = gl16(ra, p, s1);
            if (p < RB) uB[p] = gl16(rb, p, s1);
        }
        uint32_t uSA[SBD], uSB[SBD];
#pragma unroll
        for (int d = 0; d < SBD; d++) {
            uSA[d] = __builtin_amdgcn_raw_buffer_load_b32(rsa_, vsoff, s1 * 4 * SBD + 4 * d, 0);
            uSB[d] = __builtin_amdgcn_raw_buffer_load_b32(rsb_, vsoff, s1 * 4 * SBD + 4 * d, 0);
        }
#pragma unroll
        for (int p = 0; p < 8; p++) {
            swrite_a(lA0, p);
            if (p < RB) swrite_b(lB0, p);
        }
        wr_scales(lS0);
#pragma unroll
        for (int p = 0; p < 8; p++) {
            stA[p] = gl16(ra, p, min(2, nstages - 1));
            *(uint4*)(lA1 + p * 32 * BKB + wofs) = uA[p];
            if (p < RB) stB[p] = uB[p];
        }
#pragma unroll
        for (int d = 0; d < SBD; d++) {
            stSA[d] = uSA[d];
            stSB[d] = uSB[d];
        }
    }
    // stages 2 and 3 warm L2 here; the main loop warms stage s + 4
    prefetch(min(2, nstages - 1));
    prefetch(min(3, nstages - 1));
    half_barrier();
#pragma unroll
    for (int q = 0; q < 4 + JT; q++) rd_frag(F0, lA0, lB0, 0, q);
#pragma unroll
    for (int t = 0; t < 4 + JT; t++) rd_scale(F0, lS0, t, 0);

    // Stage s computes from buffer X and fills buffer Y with stage s+1 and
    // X with stage s+2.  Each k-step is a phase of 16 MFMAs from one
    // fragment set while the other set is read for the next k-step (the
    // sets alternate with the k-step's parity).  The barrier comes before
    // the last phase, which reads the next stage's first k-step from Y.
    // The LDS writes are split so that no phase carries all of them: the
    // first phase writes stage s+1's B tile to Y (its A tile went there in
    // the last phase of stage s-1) and reloads it with stage s+2, the
    // second writes the scales; the last phase, after the barrier that
    // ends every read of X, writes stage s+2's A tile to X and reloads it
    // with stage s+3.  Each register-held tile has a whole stage to arrive.
    // (Half tiles: 8 MFMAs per phase; each slot reads one fragment and its
    // scale, and the last phase writes an A run after every MFMA.)
    auto phase = [&](auto KSC, int s, Frag& cur, Frag& nxt, uint8_t* xA, const uint8_t* xB, const uint32_t* xS,
                     uint8_t* yA, uint8_t* yB, uint32_t* yS) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSC)::value;
        constexpr bool last = ks == KS - 1;
        const int s2 = min(s + 2, nstages - 1), s3 = min(s + 3, nstages - 1);
#pragma unroll
        for (int m = 0; m < NM; m++) {
            mma(cur, ks, m);
            __builtin_amdgcn_sched_barrier(0);
            const bool rf = NB == 256 ? m < 8 : m < 4 + JT;          // fragment read in this slot
            const bool rs = NB == 256 ? m >= 8 : m < 4 + JT;         // scale read in this slot
            const int qf = m, qs = NB == 256 ? m - 8 : m;
            if (rf) {
                if constexpr (last) rd_frag(nxt, yA, yB, 0, qf);
                else rd_frag(nxt, xA, xB, ks + 1, qf);
            }
            if (rs) {
                if constexpr (last) rd_scale(nxt, yS, qs, 0);
                else rd_scale(nxt, xS, qs, ks + 1);
            }
            if constexpr (ks == 0) {
                if (m < RB) {
                    swrite_b(yB, m);
                    stB[m] = gl16(rb, m, s2);
                }
                if (m == (NB == 256 ? 9 : 5)) prefetch(min(s + 4, nstages - 1));
            }
            if constexpr (ks == (KS == 2 ? 0 : 1)) {
                if (m == (NB == 256 ? 8 : 6)) {
                    wr_scales(yS);
                    gload_scales(s2);
                }
            }
            if constexpr (last) {
                const int p = NB == 256 ? m - 8 : m;
                if (p >= 0) {
                    swrite_a(xA, p);
                    stA[p] = gl16(ra, p, s3);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        pin4(acc);
        if constexpr (ks == KS - 2) half_barrier();
    };
    auto stage = [&](int s, uint8_t* xA, uint8_t* xB, uint32_t* xS, uint8_t* yA, uint8_t* yB,
                     uint32_t* yS) __attribute__((always_inline)) {
        phase(std::integral_constant<int, 0>{}, s, F0, F1, xA, xB, xS, yA, yB, yS);
        phase(std::integral_constant<int, 1>{}, s, F1, F0, xA, xB, xS, yA, yB, yS);
        if constexpr (KS == 4) {
            phase(std::integral_constant<int, 2>{}, s, F0, F1, xA, xB, xS, yA, yB, yS);
            phase(std::integral_constant<int, 3>{}, s, F1, F0, xA, xB, xS, yA, yB, yS);
        }
    };
    for (int s = 0; s < nstages; s += 2) {
        stage(s, lA0, lB0, lS0, lA1, lB1, lS1);
        if (s + 1 < nstages) stage(s + 1, lA1, lB1, lS1, lA0, lB0, lS0);
    }

    // ---- epilogue: per-tensor scales once ----
    float ap = g.alpha;
    if (g.ta) ap = ap * *g.ta;
    if (g.tb) ap = ap * *g.tb;
    if (g.hadamard_k) ap = ap * 0.03125f;
    half_barrier();                                  // every wave done with the stage buffers

    if constexpr (OUT == 1) {
        // each wave stages its 128 x NB/2 part (NB-byte rows) in LDS: 32 KiB
        // (half tiles 16 KiB, the size of a B stage buffer)
        constexpr int WC = NB / 2;                   // columns per wave
        uint8_t* buf = wave == 0 ? lA0 : wave == 1 ? lA1 : wave == 2 ? lB0 : lB1;
        uint16_t* ct = (uint16_t*)buf;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < JT; j++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {     // rows r and r + 1 of the accumulator
                    const int row = i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    const int col = j * 32 + l32;
                    const uint32_t u = f32x2_to_bf16x2_rne(acc[i][j][r] * ap, acc[i][j][r + 1] * ap);
                    ct[row * WC + col] = (uint16_t)u;
                    ct[(row + 1) * WC + col] = (uint16_t)(u >> 16);
                }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        const bool vec = (g.ldc % 8) == 0 && (((uintptr_t)g.c) & 15u) == 0;
        const int64_t rbase = m0 + wm * 128, cbase = n0 + wn * WC;
        constexpr int CPR = WC / 8;                  // 16-byte chunks per row
#pragma unroll 4
        for (int p = 0; p < 128 * CPR / 64; p++) {
            const int id = p * 64 + lane;
            const int row = id / CPR, c8 = (id % CPR) * 8;
            const int64_t grow = rbase + row, gcol = cbase + c8;
            if (grow >= g.M) continue;
            const uint4 v = *(const uint4*)(ct + row * WC + c8);
            uint16_t* dst = (uint16_t*)g.c + grow * g.ldc + gcol;
            if (vec && gcol + 8 <= g.N) {
                store_nt16(dst, v);
            } else {
                const uint16_t* e = (const uint16_t*)&v;
                for (int k = 0; k < 8; k++)
                    if (gcol + k < g.N) dst[k] = e[k];
            }
        }
    } else if constexpr (OUT >= 2) {
        // MX-quantized output (OUT 2: E4M3, 3: E5M2), 1x32 blocks along the
        // rows of C.  Each wave stages a 32-row slab of its quarter as fp32
        // in its own LDS region (rows padded to 132 floats), then each lane
        // encodes two of the slab's 128 row blocks and stores 32 code bytes
        // and one scale byte per block.
        constexpr int QF = OUT == 2 ? E4M3 : E5M2;
        constexpr int PF = 132;
        uint8_t* buf = wave == 0 ? lA0 : wave == 1 ? lA1 : wave == 2 ? lB0 : lB1;
        float* ft = (float*)buf;
        const int64_t nblk = g.N / 32;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    ft[(8 * (r / 4) + 4 * h + (r % 4)) * PF + j * 32 + l32] = acc[i][j][r] * ap;
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int b = lane + 64 * t, row = b >> 2, blk = b & 3;
                float v[32];
#pragma unroll
                for (int m = 0; m < 8; m++) {
                    const float4 x4 = *(const float4*)(ft + row * PF + blk * 32 + 4 * m);
                    v[4 * m] = x4.x; v[4 * m + 1] = x4.y; v[4 * m + 2] = x4.z; v[4 * m + 3] = x4.w;
                }
                uint32_t codes[8];
                const uint32_t sb = encode_out_block<QF>(v, codes);
                const int64_t grow = m0 + wm * 128 + i * 32 + row, gcol = n0 + wn * 128 + blk * 32;
                if (grow < g.M && gcol < g.N) {
                    uint8_t* dst = (uint8_t*)g.c + grow * g.N + gcol;
                    store_nt16(dst, make_uint4(codes[0], codes[1], codes[2], codes[3]));
                    store_nt16(dst + 16, make_uint4(codes[4], codes[5], codes[6], codes[7]));
                    g.cs[grow * nblk + gcol / 32] = (uint8_t)sb;   // cached: L2 merges the bytes of a line
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < JT; j++) {
                const int64_t col = n0 + wn * (NB / 2) + j * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (row < g.M && col < g.N) __builtin_nontemporal_store(acc[i][j][r] * ap, &((float*)g.c)[row * g.ldc + col]);
                }
            }
    }
#endif
}

int cu_count()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return cus;
}

template <int FA, int FB, int OUT>
hipError_t launch3(const GArgs& a, hipStream_t s)
{
    const unsigned nwg = (unsigned)(a.tiles_m * a.tiles_n);
    constexpr int EPB = FA == E2M1 ? 2 : 1;
    if (!a.reg_path && (a.K / EPB) % BKB == 0) {
        if constexpr (OUT < 2) {
            // Last partial round: with one 256x256 tile per CU at a time, a
            // grid of R full rounds plus r < CUs/2 tiles takes R + 1 rounds
            // of time.  When the r tiles are whole tile rows, they run as a
            // second launch of 2r half tiles (256 x 128), which takes half
            // a round.  (E.g. 6144 x 4096: 384 tiles on 256 CUs.)
            const int cus = cu_count();
            const int total = (int)nwg, r = total % cus;
            if (total > cus && r != 0 && r % a.tiles_n == 0 && 2 * r <= cus) {
                const int tr = r / a.tiles_n;
                GArgs head = a, tail = a;
                head.tiles_m = a.tiles_m - tr;
                head.M = (int64_t)head.tiles_m * BM;
                const int64_t kbytes = a.K / EPB, kblocks = a.K / 32;
                const size_t es = OUT == 1 ? 2 : 4;
                tail.qa = a.qa + head.M * kbytes;
                tail.sa = a.sa + head.M * kblocks;
                tail.c = (uint8_t*)a.c + (size_t)(head.M * a.ldc) * es;
                tail.M = a.M - head.M;
                tail.tiles_m = tr;
                tail.tiles_n = (int)((a.N + 127) / 128);
                k_gemm_w4<FA, FB, OUT, 256><<<dim3(head.tiles_m * head.tiles_n), dim3(256), 0, s>>>(head);
                k_gemm_w4<FA, FB, OUT, 128><<<dim3(tail.tiles_m * tail.tiles_n), dim3(256), 0, s>>>(tail);
                return hipGetLastError();
            }
        }
        k_gemm_w4<FA, FB, OUT, 256><<<dim3(nwg), dim3(256), 0, s>>>(a);
        return hipGetLastError();
    }
    if constexpr (OUT >= 2) {
        return hipErrorInvalidValue;          // the MX-quantized output is built on k_gemm_w4 only
    } else {
        k_gemm<FA, FB, OUT><<<dim3(nwg), dim3(512), 0, s>>>(a);
        return hipGetLastError();
    }
}

template <int FA, int FB>
hipError_t launch2(const GArgs& a, int out, hipStream_t s)
{
    switch (out) {
    case 0: return launch3<FA, FB, 0>(a, s);
    case 1: return launch3<FA, FB, 1>(a, s);
    case 2: return launch3<FA, FB, 2>(a, s);
    default: return launch3<FA, FB, 3>(a, s);
    }
}

}  // namespace

bool gemm_w4_eligible(const GemmJob& j)
{
    const int64_t kbytes = j.fa == E2M1 ? j.K / 2 : j.K;
    return kbytes % BKB == 0 && (((uintptr_t)j.sa | (uintptr_t)j.sb) & 3u) == 0;
}

hipError_t launch_gemm(const GemmJob& j, hipStream_t stream)
{
    GArgs a;
    a.qa = j.qa; a.sa = j.sa; a.ta = j.ta;
    a.qb = j.qb; a.sb = j.sb; a.tb = j.tb;
    a.M = j.M; a.N = j.N; a.K = j.K;
    a.alpha = j.alpha; a.hadamard_k = j.hadamard_k;
    a.c = j.c; a.ldc = j.ldc; a.cs = j.cs;
    a.tiles_m = (int)((j.M + BM - 1) / BM);
    a.tiles_n = (int)((j.N + BN - 1) / BN);
    a.reg_path = (((uintptr_t)j.sa | (uintptr_t)j.sb) & 3u) != 0;
    if (j.fa == E2M1) return launch2<E2M1, E2M1>(a, j.out_dtype, stream);
    if (j.fa == E4M3 && j.fb == E4M3) return launch2<E4M3, E4M3>(a, j.out_dtype, stream);
    if (j.fa == E5M2 && j.fb == E4M3) return launch2<E5M2, E4M3>(a, j.out_dtype, stream);
    if (j.fa == E4M3 && j.fb == E5M2) return launch2<E4M3, E5M2>(a, j.out_dtype, stream);
    return launch2<E5M2, E5M2>(a, j.out_dtype, stream);
}

}  // namespace mx
