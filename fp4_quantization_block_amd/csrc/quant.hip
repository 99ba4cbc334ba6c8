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
// Kernels
//   k_quant_row   row copy only: one thread per 1x32 block, read straight
//                 from global memory (64 contiguous bytes per lane for bf16),
//                 no cross-lane traffic.
//   k_quant_tile_dma / k_quant_tile_reg   column copy, or both copies from
//                 one read.  Persistent workgroups walk tiles held raw in
//                 LDS; each compute thread quantizes row and column blocks
//                 of the tile.  Column copies are stored transposed, a
//                 128-byte (FP8) run per column and tile.  The _dma form
//                 (round to nearest, 16-byte-aligned sources; tiles of 128
//                 rows x 256 source bytes) adds a loader wave that streams
//                 tiles two ahead into three LDS buffers with direct loads;
//                 the _reg form (stochastic rounding, or any alignment;
//                 128 x 64 tiles) prefetches the next tile into registers.
//                 For stochastic rounding of column blocks the workgroup
//                 generates the tile's Philox words into LDS, four per
//                 call, so no word is wasted.
//   k_amax_partial / k_amax_reduce   level-1 tensor amax for the two-level
//                 scheme: per-workgroup partial maxima, then one workgroup
//                 writes s_t = amax / Fmax.  The partials are parked in the
//                 caller's scale array, which the quantize kernel overwrites
//                 afterwards (no atomics, no extra memory).
#include <mutex>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

constexpr int TR = 128, TC = 64;           // quantizer tile (rows x columns)

template <int SRC> struct SrcT;
template <> struct SrcT<SRC_BF16> { static constexpr int bytes = 2; };
template <> struct SrcT<SRC_F32> { static constexpr int bytes = 4; };

typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

struct QArgs {
    const void* x;
    int64_t rows, cols, ld;
    uint8_t* q_row; uint8_t* s_row;
    uint8_t* q_col; uint8_t* s_col;
    const float* tscale;          // s_t (two-level), read by the quantize kernels
    uint32_t k0, k1, offset;
    int hadamard, two_level;
    int vec;                      // 1: x and every row start are 16-byte aligned
    int64_t ntx, ntiles;          // tiles per tile row, tile count
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

// The 32 values of one block ready for the block scale: source values from
// elem(i), divided by s_t (two-level) and transformed (Hadamard).  Returns the
// block's |max| key.
template <class Elem>
__device__ __forceinline__ uint32_t block_values(Elem&& elem, bool two_level, bool had,
                                                 const TensorDiv& d, float (&v)[32])
{
#pragma unroll
    for (int i = 0; i < 32; i++) v[i] = elem(i);
    uint32_t key = 0;
    bool have = false;
    if (two_level) {
        bool slow = !d.fast;
        if (d.fast) {
            uint32_t lo = ~0u, qk = 0;
#pragma unroll
            for (int i = 0; i < 32; i++) {
                v[i] = div_fast(v[i], d, lo);
                qk = max(qk, abs_key(v[i]));
            }
            slow = lo < d.lo_key || (qk > 0x48000000u && qk < 0x7F800000u);   // 0x48000000 = 2^17
            key = qk;
        }
        if (slow) {
            key = 0;
#pragma unroll
            for (int i = 0; i < 32; i++) {
                v[i] = elem(i) / d.s;
                key = max(key, abs_key(v[i]));
            }
        }
        have = true;
    }
    if (had) {
        key = fwht32_key(v);
        have = true;
    }
    if (!have) {
        key = 0;
#pragma unroll
        for (int i = 0; i < 32; i++) key = max(key, abs_key(v[i]));
    }
    return key;
}

// |max| key of 32 bf16 values held as 16 packed dwords (packed 16-bit max)
__device__ __forceinline__ uint32_t bf16_block_key(const uint32_t* w)
{
    ushort2v m = {0, 0};
#pragma unroll
    for (int j = 0; j < 16; j++) m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2v, w[j] & 0x7FFF7FFFu));
    return (uint32_t)max(m.x, m.y) << 16;
}

// Encodes one block whose 32 values v have the |max| key `key`.  words(k)
// returns the random words of elements 4k..4k+3 (SR only).  Writes 8 (FP8)
// or 4 (FP4) dwords of packed codes; returns the scale byte.  A block
// holding a NaN or Inf gets byte 0xFF and the canonical NaN code 0x7F for
// every element (E2M1, which has no NaN: 0) -- IEEE 754 leaves the sign of a
// NaN produced by arithmetic undefined, so no sign is carried.
template <int FMT, bool SR, class Words>
__device__ __forceinline__ uint32_t encode_block(const float (&v)[32], uint32_t key, Words&& words,
                                                 uint32_t* out)
{
    constexpr int BITS = Fmt<FMT>::bits;
    if (key >= 0x7F800000u) {
#pragma unroll
        for (int k = 0; k < (BITS == 8 ? 8 : 4); k++) out[k] = BITS == 8 ? 0x7F7F7F7Fu : 0u;
        return 0xFFu;
    }
    const int e = block_exponent<FMT>(key);
    float y[32];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        u32x4 w{0u, 0u, 0u, 0u};
        if constexpr (SR) w = words(k);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float t = scale_by(v[4 * k + j], e);
            y[4 * k + j] = SR ? sr_value<FMT>(t, u[j]) : clamp_fmax<FMT>(t);
        }
    }
    if constexpr (BITS == 8) {
#pragma unroll
        for (int k = 0; k < 8; k++) out[k] = cvt4_fp8<FMT>(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; k++) out[k] = cvt8_fp4(&y[8 * k]);
    }
    return (uint32_t)(e + 127);
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* dst, const uint32_t* w)
{
    *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
    if constexpr (BITS == 8) *(uint4*)(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
}

// raw bits of source element i (bf16 in the low 16 bits)
template <int SRC>
__device__ __forceinline__ uint32_t raw1(const void* x, int64_t i)
{
    if constexpr (SRC == SRC_BF16) return ((const uint16_t*)x)[i];
    else return ((const uint32_t*)x)[i];
}

// source value from a raw dword array: element i of bf16 pairs or fp32 words
template <int SRC>
__device__ __forceinline__ float unpack(const uint32_t* w, int i)
{
    if constexpr (SRC == SRC_BF16) return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    else return __uint_as_float(w[i]);
}

// the four row-stream (axis 0) words of elements 4(n0 + k) .. 4(n0 + k) + 3
struct RowWords {
    uint64_t n0; uint32_t offset, k0, k1;
    __device__ __forceinline__ u32x4 operator()(int k) const
    {
        return philox_block(n0 + (uint64_t)k, 0u, offset, k0, k1);
    }
};

// ---------------------------------------------------------------------------
// Row copy: one thread per 1x32 block.  Grid: x covers the blocks of a row
// in runs of 64 (one per lane), y covers rows four at a time (one per wave).
// ---------------------------------------------------------------------------
template <int SRC, int FMT, bool SR>
__global__ __launch_bounds__(256) void k_quant_row(QArgs a)
{
    constexpr int BITS = Fmt<FMT>::bits;
    constexpr int NW = SRC == SRC_BF16 ? 16 : 32;      // source dwords per block
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nblk = a.cols / 32;
    const int64_t cb = (int64_t)blockIdx.x * 64 + lane;
    if (cb >= nblk) return;
    const TensorDiv d = make_div(a.two_level ? *a.tscale : 1.0f);
    for (int64_t r = (int64_t)blockIdx.y * 4 + wave; r < a.rows; r += (int64_t)gridDim.y * 4) {
        const int64_t base = r * a.ld + cb * 32;
        uint32_t w[NW];
        if (a.vec) {
            const uint4* p = (const uint4*)((const uint8_t*)a.x + base * SrcT<SRC>::bytes);
#pragma unroll
            for (int k = 0; k < NW / 4; k++) {
                const uint4 t = p[k];
                w[4 * k] = t.x; w[4 * k + 1] = t.y; w[4 * k + 2] = t.z; w[4 * k + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NW; j++)
                w[j] = SRC == SRC_BF16 ? raw1<SRC>(a.x, base + 2 * j) | (raw1<SRC>(a.x, base + 2 * j + 1) << 16)
                                       : raw1<SRC>(a.x, base + j);
        }
        float v[32];
        uint32_t key;
        if (SRC == SRC_BF16 && !a.two_level && !a.hadamard) {
#pragma unroll
            for (int i = 0; i < 32; i++) v[i] = unpack<SRC>(w, i);
            key = bf16_block_key(w);
        } else {
            key = block_values([&](int i) { return unpack<SRC>(w, i); }, a.two_level, a.hadamard, d, v);
        }
        const RowWords words{((uint64_t)r * (uint64_t)a.cols + (uint64_t)(cb * 32)) >> 2, a.offset, a.k0, a.k1};
        uint32_t codes[8];
        const uint32_t sb = encode_block<FMT, SR>(v, key, words, codes);
        store_codes<BITS>(a.q_row + r * (a.cols * BITS / 8) + cb * 32 * BITS / 8, codes);
        a.s_row[r * nblk + cb] = (uint8_t)sb;
    }
}

// ---------------------------------------------------------------------------
// Column copy (and optionally the row copy) through LDS-staged tiles of
// TR x TC source elements.  Two LDS layouts of a tile:
//   PadLayout  rows padded by 16 bytes (tiles written from registers);
//   SwzLayout  dense rows whose 16-byte chunks are XOR-permuted by a key of
//              the row (tiles written by direct global->LDS loads, which fill
//              1 KiB of consecutive LDS per instruction).
// Both keep the row-block reads (16 consecutive rows, ds_read_b128) and the
// column reads (64 consecutive columns of one row) free of bank conflicts.
// ---------------------------------------------------------------------------
template <int SRC> struct PadLayout {
    static constexpr int RB = TC * SrcT<SRC>::bytes, PITCH = RB + 16, BYTES = TR * PITCH;
    __device__ static int at(int row, int byte) { return row * PITCH + byte; }
};
template <int SRC> struct SwzLayout {
    static constexpr int RB = TC * SrcT<SRC>::bytes, BYTES = TR * RB;
    __device__ static int key(int row) { return SRC == SRC_BF16 ? (row >> 1) & 7 : row & 15; }
    __device__ static int at(int row, int byte)
    {
        return row * RB + ((((byte >> 4) ^ key(row)) << 4) | (byte & 15));
    }
};

// Quantizes the tile at (r0, c0) held in LDS: one row block (ROW) and one
// column block per thread of the 256 compute threads; for SR the column words
// are generated into `words` first.  words_ready() is the workgroup barrier
// between generating and reading them.
template <int SRC, int FMT, bool ROW, bool SR, class L, class Sync>
__device__ __forceinline__ void quantize_tile(const QArgs& a, const TensorDiv& d, const uint8_t* tile,
                                              uint32_t* words, int64_t r0, int64_t c0, int nrow, int ncol,
                                              int tid, Sync&& words_ready)
{
    constexpr int EB = SrcT<SRC>::bytes;
    constexpr int BITS = Fmt<FMT>::bits;
    if constexpr (SR) {
        if ((a.cols & 3) == 0) {                // one call per 4 consecutive columns
#pragma unroll
            for (int p = 0; p < TR * TC / 4 / 256; p++) {
                const int id = p * 256 + tid;
                const int r = id / (TC / 4), c4 = (id % (TC / 4)) * 4;
                if (r < nrow && c4 < ncol) {
                    const uint64_t idx = (uint64_t)(r0 + r) * (uint64_t)a.cols + (uint64_t)(c0 + c4);
                    const u32x4 w = philox_block(idx >> 2, 1u, a.offset, a.k0, a.k1);
                    *(uint4*)&words[r * TC + c4] = make_uint4(w.x, w.y, w.z, w.w);
                }
            }
        } else {                                // general: one call per element
            for (int p = 0; p < TR * TC / 256; p++) {
                const int id = p * 256 + tid;
                const int r = id / TC, c = id % TC;
                if (r < nrow && c < ncol) {
                    const uint64_t idx = (uint64_t)(r0 + r) * (uint64_t)a.cols + (uint64_t)(c0 + c);
                    words[r * TC + c] = pick(philox_block(idx >> 2, 1u, a.offset, a.k0, a.k1), (uint32_t)(idx & 3));
                }
            }
        }
    }

    // ---- row block: thread -> (row tid % 128, block tid / 128) ----
    if constexpr (ROW) {
        const int r = tid % TR, h = tid / TR;
        if (r < nrow && h * 32 < ncol) {
            constexpr int NW = 32 * EB / 4;
            uint32_t w[NW];
#pragma unroll
            for (int k = 0; k < NW / 4; k++) {
                const uint4 q = *(const uint4*)&tile[L::at(r, h * 32 * EB + 16 * k)];
                w[4 * k] = q.x; w[4 * k + 1] = q.y; w[4 * k + 2] = q.z; w[4 * k + 3] = q.w;
            }
            float v[32];
            uint32_t key;
            if (SRC == SRC_BF16 && !a.two_level && !a.hadamard) {
#pragma unroll
                for (int i = 0; i < 32; i++) v[i] = unpack<SRC>(w, i);
                key = bf16_block_key(w);
            } else {
                key = block_values([&](int i) { return unpack<SRC>(w, i); }, a.two_level, a.hadamard, d, v);
            }
            const int64_t gc = c0 + h * 32;
            const RowWords rw{((uint64_t)(r0 + r) * (uint64_t)a.cols + (uint64_t)gc) >> 2, a.offset, a.k0, a.k1};
            uint32_t codes[8];
            const uint32_t sb = encode_block<FMT, SR>(v, key, rw, codes);
            store_codes<BITS>(a.q_row + (r0 + r) * (a.cols * BITS / 8) + gc * BITS / 8, codes);
            a.s_row[(r0 + r) * (a.cols / 32) + gc / 32] = (uint8_t)sb;
        }
    }
    if constexpr (SR) words_ready();

    // ---- column block: thread -> (column tid % 64, row block tid / 64) ----
    const int c = tid % TC, rb = tid / TC;
    if (c < ncol && rb * 32 < nrow) {
        auto elem = [&](int i) {
            const uint8_t* p = &tile[L::at(rb * 32 + i, c * EB)];
            if constexpr (SRC == SRC_BF16) return __uint_as_float((uint32_t)*(const uint16_t*)p << 16);
            else return *(const float*)p;
        };
        float v[32];
        const uint32_t key = block_values(elem, a.two_level, a.hadamard, d, v);
        auto cw = [&](int k) {
            const uint32_t* p = &words[(rb * 32 + 4 * k) * TC + c];
            return u32x4{p[0], p[TC], p[2 * TC], p[3 * TC]};
        };
        uint32_t codes[8];
        const uint32_t sb = encode_block<FMT, SR>(v, key, cw, codes);
        const int64_t gc = c0 + c, gr = r0 + rb * 32;
        store_codes<BITS>(a.q_col + gc * (a.rows * BITS / 8) + gr * BITS / 8, codes);
        a.s_col[gc * (a.rows / 32) + gr / 32] = (uint8_t)sb;
    }
}

// The k-th tile (TRR x TCC) of this workgroup's sequence ((r0, c0) of its
// corner), or false past the end.  Workgroups are dealt to the 8 XCDs
// round-robin; when the grid allows, XCD j walks its own strip of tile
// columns (row-major inside the strip), so the partial lines of both output
// copies -- a row's code and scale bytes, a column's scale bytes -- are
// completed inside one XCD's L2 instead of being merged in memory.
template <int TRR, int TCC>
__device__ __forceinline__ bool tile_at(const QArgs& a, int64_t k, int64_t& r0, int64_t& c0)
{
    const int64_t nty = a.ntiles / a.ntx;
    if (a.ntx >= 8 && (gridDim.x & 7) == 0) {
        const int64_t j = blockIdx.x & 7, l = blockIdx.x >> 3, L = gridDim.x >> 3;
        const int64_t x0 = j * a.ntx / 8, x1 = (j + 1) * a.ntx / 8, width = x1 - x0;
        const int64_t s = l + k * L;
        if (s >= width * nty) return false;
        r0 = (s / width) * TRR;
        c0 = (x0 + s % width) * TCC;
        return true;
    }
    const int64_t t = blockIdx.x + k * (int64_t)gridDim.x;
    if (t >= a.ntiles) return false;
    r0 = (t / a.ntx) * TRR;
    c0 = (t % a.ntx) * TCC;
    return true;
}

template <int TRR, int TCC>
__device__ __forceinline__ void tile_extent(const QArgs& a, int64_t r0, int64_t c0, int& nrow, int& ncol)
{
    nrow = (int)(a.rows - r0 < TRR ? a.rows - r0 : TRR);      // a multiple of 32
    ncol = (int)(a.cols - c0 < TCC ? a.cols - c0 : TCC);
}

// Barrier for LDS hand-offs without a memory fence: waits only for this
// wave's LDS traffic (not for its global stores), then s_barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Same for the loader wave: its direct-to-LDS loads have landed.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// k_quant_tile_dma: 16-byte-aligned sources, round to nearest.  Tiles of
// 128 rows x 256 source bytes (128 bf16 or 64 fp32 columns).  NCW compute
// waves plus one loader wave: the loader streams tiles two ahead into three
// LDS tile buffers (direct global->LDS buffer loads of 16 bytes per lane;
// rows past the tensor read as zero, columns past it hold neighbouring data
// or zeros, and neither is used) while the compute waves quantize the
// current one, so the compute waves never wait on a global load and the
// loader never waits on a store.  Codes are staged in an LDS buffer of their
// own, then written out as whole runs:
// each column's codes for the tile form one 128-byte (FP8) or 64-byte (FP4)
// run of the transposed copy, each row's one run of the row copy, and scale
// bytes leave four to a store.  Two barriers per tile: one when every block
// of the tile has been read (its buffer is then free for the loader), one
// when the codes are staged and the next tile has landed.  Scattered 16- to
// 32-byte stores (one per block) were measured at under 2.2 TB/s on this
// part; whole runs reach the
// HBM rate.
// ---------------------------------------------------------------------------
template <int SRC> struct DmaTile {
    static constexpr int EB = SrcT<SRC>::bytes, ROWS = 128, COLS = 256 / EB, RB = 256;
    // dense 256-byte rows whose 16-byte chunks are XOR-permuted by the row
    // (chunk c of row r sits at position c ^ (r & 15)): 16 consecutive rows
    // read with ds_read_b128 at one chunk hit 16 different bank groups, a
    // row read by consecutive lanes stays inside its row, and four rows
    // form one contiguous 1 KiB run, the unit of a 16-byte-per-lane direct
    // load
    static constexpr int BYTES = ROWS * RB;
    // compute waves: one column block and one row block per thread for bf16
    static constexpr int NCW = SRC == SRC_BF16 ? 8 : 4;
    __device__ static int at(int row, int byte) { return row * RB + ((((byte >> 4) ^ (row & 15))) << 4) + (byte & 15); }
};

// loader wait at the end of a tile when the tile after next is in flight:
// all but its 32 direct loads (the next tile's) complete, then the barrier
__device__ __forceinline__ void dma_barrier_keep32() { asm volatile("s_waitcnt vmcnt(32)\n\ts_barrier" ::: "memory"); }

// Output staging of LB-byte lines (LB = 32, 64 or 128): the 16-byte chunks of
// a line are XOR-permuted so that 16 lanes writing one chunk of 16
// consecutive lines, or reading consecutive chunks, hit distinct banks.
template <int LB>
__device__ __forceinline__ int stage_at(int line, int chunk)
{
    constexpr int CH = LB / 16, LPR = 256 / LB;
    return line * LB + ((chunk ^ ((line / LPR) % CH)) << 4);
}

// n scale bytes (n <= 4) from a staged dword to dst: one store when aligned
__device__ __forceinline__ void store_scales(uint8_t* dst, uint32_t w, int n)
{
    if (n == 4 && (reinterpret_cast<uintptr_t>(dst) & 3u) == 0) {
        *(uint32_t*)dst = w;
    } else if (n == 2 && (reinterpret_cast<uintptr_t>(dst) & 1u) == 0) {
        *(uint16_t*)dst = (uint16_t)w;
    } else {
        for (int i = 0; i < n; i++) dst[i] = (uint8_t)(w >> (8 * i));
    }
}

template <int SRC, int FMT, bool ROW>
__global__ __launch_bounds__(64 * (DmaTile<SRC>::NCW + 1)) void k_quant_tile_dma(QArgs a)
{
    using T = DmaTile<SRC>;
    constexpr int EB = T::EB, TRR = T::ROWS, TCC = T::COLS, NCT = 64 * T::NCW;
    constexpr int BITS = Fmt<FMT>::bits, CW = BITS == 8 ? 8 : 4;   // code dwords per block
    constexpr int LBC = TRR * BITS / 8;         // bytes of one column's codes per tile
    constexpr int LBR = TCC * BITS / 8;         // bytes of one row's codes per tile
    constexpr int NT = TRR * TCC / 32 / NCT;    // column (and row) blocks per compute thread
    constexpr int SPR = TCC / 32;               // row scale bytes per tile row
    static_assert(NT >= 1 && TRR * TCC / 32 == NT * NCT, "tile / thread split");
    // three tile buffers: tile k is read while k+1 lands and k+2 is loading;
    // the codes are staged in a buffer of their own, so a tile buffer is free
    // for the loader as soon as its blocks have been read
    __shared__ __align__(16) uint8_t buf0[T::BYTES];
    __shared__ __align__(16) uint8_t buf1[T::BYTES];
    __shared__ __align__(16) uint8_t buf2[T::BYTES];
    __shared__ __align__(16) uint8_t stg[TCC * LBC + TRR * LBR];
    __shared__ __align__(4) uint8_t sc_col[TCC * 4];
    __shared__ __align__(4) uint8_t sc_row[TRR * SPR];

    const int tid = threadIdx.x;
    if (tid >= NCT) {
        // ---------------- loader wave ----------------
        // 32 direct loads per tile, 16 bytes per lane: load p fills the
        // contiguous 1 KiB of tile rows 4p .. 4p+3; lane l writes LDS chunk
        // position l % 16 of row 4p + l / 16, i.e. source chunk
        // (l % 16) ^ (row & 15).  The row offset is part of the range-checked
        // lane offset, so rows past the tensor (and, with cols * elem a
        // multiple of 16, bytes past its end) read as zero.
        const int l = tid - NCT;
        const uint32_t lrow = (uint32_t)(l >> 4), lcp = (uint32_t)(l & 15);
        auto issue = [&](int64_t r0, int64_t c0, uint8_t* dst) {
            int64_t n = ((a.rows - r0 - 1) * a.ld + (a.cols - c0)) * EB;
            n = n > 0xFFFFFFFFll ? 0xFFFFFFFFll : n;
            const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((const uint8_t*)a.x + (r0 * a.ld + c0) * EB), (short)0, (int)(uint32_t)n, 0x00020000);
            const uint32_t row_bytes = (uint32_t)(a.ld * EB);
#pragma unroll 8
            for (int p = 0; p < TRR / 4; p++) {
                const uint32_t row = 4 * p + lrow;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + p * 1024), 16,
                                                         row * row_bytes + ((lcp ^ (row & 15)) << 4), 0, 0, 0);
            }
        };
        int64_t r0, c0, r1, c1;
        if (tile_at<TRR, TCC>(a, 0, r0, c0)) issue(r0, c0, buf0);
        if (tile_at<TRR, TCC>(a, 1, r1, c1)) {
            issue(r1, c1, buf1);
            dma_barrier_keep32();                          // tile 0 landed
        } else {
            dma_barrier();
        }
        for (int64_t k = 0; tile_at<TRR, TCC>(a, k, r0, c0); k++) {
            // tile k+2 goes to the buffer of tile k-1, free since every block
            // of tile k-1 was read
            int64_t r2, c2;
            const bool next2 = tile_at<TRR, TCC>(a, k + 2, r2, c2);
            if (next2) {
                const int m = (int)((k + 2) % 3);
                issue(r2, c2, m == 0 ? buf0 : m == 1 ? buf1 : buf2);
            }
            lds_barrier();                                // compute: tile k read
            if (next2) dma_barrier_keep32();              // codes staged; tile k+1 landed
            else dma_barrier();
        }
        return;
    }
    // ---------------- compute waves ----------------
    const TensorDiv d = make_div(a.two_level ? *a.tscale : 1.0f);
    const auto none = [](int) { return u32x4{0u, 0u, 0u, 0u}; };
    lds_barrier();
    int64_t r0, c0;
    for (int64_t k = 0; tile_at<TRR, TCC>(a, k, r0, c0); k++) {
        const int km = (int)(k % 3);
        uint8_t* tile = km == 0 ? buf0 : km == 1 ? buf1 : buf2;
        int nrow, ncol;
        tile_extent<TRR, TCC>(a, r0, c0, nrow, ncol);
        uint32_t ccode[NT][CW], csc[NT], rcode[NT][CW], rsc[NT];

        // column blocks: q -> (column q % TCC, row block q / TCC)
#pragma unroll
        for (int j = 0; j < NT; j++) {
            const int q = tid + NCT * j, c = q % TCC, rb = q / TCC;
            if (c < ncol && rb * 32 < nrow) {
                auto elem = [&](int i) {
                    const uint8_t* p = &tile[T::at(rb * 32 + i, c * EB)];
                    if constexpr (SRC == SRC_BF16) return __uint_as_float((uint32_t)*(const uint16_t*)p << 16);
                    else return *(const float*)p;
                };
                float v[32];
                const uint32_t key = block_values(elem, a.two_level, a.hadamard, d, v);
                csc[j] = encode_block<FMT, false>(v, key, none, ccode[j]);
            }
        }
        // row blocks: q -> (row q % TRR, block q / TRR)
        if constexpr (ROW) {
#pragma unroll
            for (int j = 0; j < NT; j++) {
                const int q = tid + NCT * j, r = q % TRR, blk = q / TRR;
                if (r < nrow && blk * 32 < ncol) {
                    constexpr int NW = 32 * EB / 4;
                    uint32_t w[NW];
#pragma unroll
                    for (int m = 0; m < NW / 4; m++) {
                        const uint4 t4 = *(const uint4*)&tile[T::at(r, blk * 32 * EB + 16 * m)];
                        w[4 * m] = t4.x; w[4 * m + 1] = t4.y; w[4 * m + 2] = t4.z; w[4 * m + 3] = t4.w;
                    }
                    float v[32];
                    uint32_t key;
                    if (SRC == SRC_BF16 && !a.two_level && !a.hadamard) {
#pragma unroll
                        for (int i = 0; i < 32; i++) v[i] = unpack<SRC>(w, i);
                        key = bf16_block_key(w);
                    } else {
                        key = block_values([&](int i) { return unpack<SRC>(w, i); }, a.two_level, a.hadamard, d, v);
                    }
                    rsc[j] = encode_block<FMT, false>(v, key, none, rcode[j]);
                }
            }
        }
        // every block of the tile has been read, and every wave's reads of
        // the previous tile's staged codes have completed
        lds_barrier();

        // stage codes and scales (column runs first, then row runs)
        uint8_t* scol = stg;
        uint8_t* srow = stg + TCC * LBC;
#pragma unroll
        for (int j = 0; j < NT; j++) {
            const int q = tid + NCT * j, c = q % TCC, rb = q / TCC;
            if (c < ncol && rb * 32 < nrow) {
#pragma unroll
                for (int m = 0; m < CW / 4; m++)
                    *(uint4*)&scol[stage_at<LBC>(c, rb * (CW / 4) + m)] =
                        make_uint4(ccode[j][4 * m], ccode[j][4 * m + 1], ccode[j][4 * m + 2], ccode[j][4 * m + 3]);
                sc_col[c * 4 + rb] = (uint8_t)csc[j];
            }
        }
        if constexpr (ROW) {
#pragma unroll
            for (int j = 0; j < NT; j++) {
                const int q = tid + NCT * j, r = q % TRR, blk = q / TRR;
                if (r < nrow && blk * 32 < ncol) {
#pragma unroll
                    for (int m = 0; m < CW / 4; m++)
                        *(uint4*)&srow[stage_at<LBR>(r, blk * (CW / 4) + m)] =
                            make_uint4(rcode[j][4 * m], rcode[j][4 * m + 1], rcode[j][4 * m + 2], rcode[j][4 * m + 3]);
                    sc_row[r * SPR + blk] = (uint8_t)rsc[j];
                }
            }
        }
        lds_barrier();                                   // staging complete; tile k+1 landed

        // whole runs out (the next tile's reads of its own buffer follow
        // without a barrier)
        const int64_t colbytes = a.rows * BITS / 8, rowbytes = a.cols * BITS / 8;
        for (int id = tid; id < TCC * (LBC / 16); id += NCT) {
            const int line = id / (LBC / 16), ch = id % (LBC / 16);
            if (line < ncol && ch * 16 < nrow * BITS / 8)
                *(uint4*)(a.q_col + (c0 + line) * colbytes + r0 * BITS / 8 + ch * 16) =
                    *(const uint4*)&scol[stage_at<LBC>(line, ch)];
        }
        if constexpr (ROW) {
            for (int id = tid; id < TRR * (LBR / 16); id += NCT) {
                const int line = id / (LBR / 16), ch = id % (LBR / 16);
                if (line < nrow && ch * 16 < ncol * BITS / 8)
                    *(uint4*)(a.q_row + (r0 + line) * rowbytes + c0 * BITS / 8 + ch * 16) =
                        *(const uint4*)&srow[stage_at<LBR>(line, ch)];
            }
        }
        if (tid < ncol)
            store_scales(a.s_col + (c0 + tid) * (a.rows / 32) + r0 / 32, *(const uint32_t*)&sc_col[tid * 4], nrow / 32);
        if constexpr (ROW) {
            const int r = tid - (NCT - TRR);                 // the last TRR compute threads
            if (r >= 0 && r < nrow) {
                uint32_t w = 0;
#pragma unroll
                for (int i = 0; i < SPR; i++) w |= (uint32_t)sc_row[r * SPR + i] << (8 * i);
                store_scales(a.s_row + (r0 + r) * (a.cols / 32) + c0 / 32, w, ncol / 32);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_quant_tile_reg: any alignment.  Persistent workgroups; the next tile is
// loaded into registers (element by element where needed) while the current
// one is quantized, then written to a padded LDS tile.
// ---------------------------------------------------------------------------
template <int SRC, int FMT, bool ROW, bool SR>
__global__ __launch_bounds__(256) void k_quant_tile_reg(QArgs a)
{
    using L = PadLayout<SRC>;
    constexpr int EB = SrcT<SRC>::bytes;
    constexpr int CPR = L::RB / 16;             // 16-byte chunks per tile row
    constexpr int NLD = TR * CPR / 256;         // chunks per thread
    constexpr int EPC = 16 / EB;                // elements per chunk
    __shared__ __align__(16) uint8_t tile[L::BYTES];
    extern __shared__ __align__(16) uint32_t words[];

    const int tid = threadIdx.x;
    const TensorDiv d = make_div(a.two_level ? *a.tscale : 1.0f);
    uint4 pre[NLD];

    auto load = [&](int64_t r0, int64_t c0) {
        int nrow, ncol;
        tile_extent<TR, TC>(a, r0, c0, nrow, ncol);
#pragma unroll
        for (int p = 0; p < NLD; p++) {
            const int id = p * 256 + tid;
            const int r = id / CPR, cc = (id % CPR) * EPC;
            const int64_t e0 = (r0 + r) * a.ld + c0 + cc;
            if (a.vec && r < nrow && cc + EPC <= ncol) {
                pre[p] = *(const uint4*)((const uint8_t*)a.x + e0 * EB);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < EPC; k++)
                    if (r < nrow && cc + k < ncol) {
                        if constexpr (SRC == SRC_BF16) w[k >> 1] |= raw1<SRC>(a.x, e0 + k) << (16 * (k & 1));
                        else w[k] = raw1<SRC>(a.x, e0 + k);
                    }
                pre[p] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };

    int64_t r0, c0;
    if (tile_at<TR, TC>(a, 0, r0, c0)) load(r0, c0);
    for (int64_t k = 0; tile_at<TR, TC>(a, k, r0, c0); k++) {
#pragma unroll
        for (int p = 0; p < NLD; p++) {
            const int id = p * 256 + tid;
            *(uint4*)&tile[L::at(id / CPR, (id % CPR) * 16)] = pre[p];
        }
        int nrow, ncol;
        tile_extent<TR, TC>(a, r0, c0, nrow, ncol);
        __syncthreads();
        int64_t r1, c1;
        if (tile_at<TR, TC>(a, k + 1, r1, c1)) load(r1, c1);      // in flight while this tile is quantized
        quantize_tile<SRC, FMT, ROW, SR, L>(a, d, tile, words, r0, c0, nrow, ncol, tid,
                                            [] { __syncthreads(); });
        __syncthreads();                                  // tile (and words) free for the next tile
    }
}

// ---------------------------------------------------------------------------
// Level-1 tensor amax (two-level scheme)
// ---------------------------------------------------------------------------
// max |x| key of the 8 (bf16) or 4 (fp32) elements of a 16-byte word
template <int SRC>
__device__ __forceinline__ uint32_t key16(uint4 w)
{
    if constexpr (SRC == SRC_BF16) {
        const uint32_t m = max(max(max(w.x & 0x7FFFu, (w.x >> 16) & 0x7FFFu),
                                   max(w.y & 0x7FFFu, (w.y >> 16) & 0x7FFFu)),
                               max(max(w.z & 0x7FFFu, (w.z >> 16) & 0x7FFFu),
                                   max(w.w & 0x7FFFu, (w.w >> 16) & 0x7FFFu)));
        return m << 16;
    } else {
        return max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu));
    }
}

template <int SRC>
__device__ __forceinline__ uint32_t key1(const void* x, int64_t i)
{
    if constexpr (SRC == SRC_BF16) return ((uint32_t)((const uint16_t*)x)[i] << 16) & 0x7FFFFFFFu;
    else return ((const uint32_t*)x)[i] & 0x7FFFFFFFu;
}

// Per-workgroup |x| keys (integer max: NaN keys exceed Inf, Inf exceeds every
// finite value).  Dense 16-byte-aligned tensors are read as a flat run of
// 16-byte words with several loads in flight; other layouts row by row.
template <int SRC>
__device__ __forceinline__ void amax_partial(const void* x, int64_t rows, int64_t cols, int64_t ld, int flat16,
                                             uint32_t* partial, int bid, int nblk)
{
    uint32_t key = 0;
    const int64_t stride = (int64_t)nblk * blockDim.x;
    const int64_t t0 = (int64_t)bid * blockDim.x + threadIdx.x;
    if (flat16) {
        constexpr int EPW = SRC == SRC_BF16 ? 8 : 4;
        const int64_t nw = rows * cols / EPW;            // whole 16-byte words
        const uint4* p = (const uint4*)x;
        int64_t i = t0;
        for (; i + 7 * stride < nw; i += 8 * stride) {   // eight loads in flight
            uint4 w[8];
#pragma unroll
            for (int k = 0; k < 8; k++) w[k] = p[i + k * stride];
#pragma unroll
            for (int k = 0; k < 8; k++) key = max(key, key16<SRC>(w[k]));
        }
        for (; i < nw; i += stride) key = max(key, key16<SRC>(p[i]));
        for (int64_t e = nw * EPW + t0; e < rows * cols; e += stride) key = max(key, key1<SRC>(x, e));
    } else {
        for (int64_t r = bid; r < rows; r += nblk)
            for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) key = max(key, key1<SRC>(x, r * ld + c));
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) partial[bid] = max(max(red[0], red[1]), max(red[2], red[3]));
}

template <int SRC>
__global__ __launch_bounds__(256) void k_amax_partial(const void* x, int64_t rows, int64_t cols,
                                                      int64_t ld, int flat16, uint32_t* partial)
{
    amax_partial<SRC>(x, rows, cols, ld, flat16, partial, blockIdx.x, gridDim.x);
}

// partial maxima of two same-shaped tensors in one launch: workgroups
// [0, n0) take x0 into p0, the rest x1 into p1
template <int SRC>
__global__ __launch_bounds__(256) void k_amax_partial2(const void* x0, int64_t ld0, int flat0, uint32_t* p0, int n0,
                                                       const void* x1, int64_t ld1, int flat1, uint32_t* p1,
                                                       int64_t rows, int64_t cols)
{
    const int b = blockIdx.x;
    if (b < n0) amax_partial<SRC>(x0, rows, cols, ld0, flat0, p0, b, n0);
    else amax_partial<SRC>(x1, rows, cols, ld1, flat1, p1, b - n0, gridDim.x - n0);
}

// One workgroup: s_t from the partial keys, written to the tensor-scale word
// (which may itself hold the single partial of a tiny tensor).
template <int FMT>
__global__ __launch_bounds__(256) void k_amax_reduce(const uint32_t* partial, int n, float* ts)
{
    uint32_t key = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) key = max(key, partial[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, m));
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) *ts = tensor_scale_from_key<FMT>(max(max(red[0], red[1]), max(red[2], red[3])));
}

// MOSS weight auto-scaling ([MOSS, "创新 2：权重自动缩放"]): one workgroup
// reduces the partial maxima of W and of g and writes the predicted scale
// (max|W| + lr * max|g|) / Fmax -- product, sum and division each rounded
// once in fp32, as written; contraction is switched off so the compiler
// cannot fuse the product into the sum (HIP contracts by default, which
// changes the last bit).  NaN when either tensor holds one.
template <int FMT>
__global__ __launch_bounds__(256) void k_predict_scale(const uint32_t* pw, int nw, const uint32_t* pg, int ng,
                                                       float lr, float* out)
{
    uint32_t kw = 0, kg = 0;
    for (int i = threadIdx.x; i < nw; i += blockDim.x) kw = max(kw, pw[i]);
    for (int i = threadIdx.x; i < ng; i += blockDim.x) kg = max(kg, pg[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        kw = max(kw, (uint32_t)__shfl_xor((int)kw, m));
        kg = max(kg, (uint32_t)__shfl_xor((int)kg, m));
    }
    __shared__ uint32_t red[2][4];
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = kw;
        red[1][threadIdx.x >> 6] = kg;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        kw = max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3]));
        kg = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
        if (kw > 0x7F800000u || kg > 0x7F800000u) {
            *out = __uint_as_float(0x7FC00000u);
            return;
        }
        float pmax;
        {
#pragma clang fp contract(off)
            const float step = lr * __uint_as_float(kg);
            pmax = __uint_as_float(kw) + step;
        }
        *out = tensor_scale_from_key<FMT>(__float_as_uint(pmax));
    }
}

// persistent grid: as many workgroups as stay resident together (at most 4
// per CU), never more than there are tiles
template <int SRC, int FMT, bool ROW, bool SR>
hipError_t launch_tile(QArgs a, hipStream_t stream)
{
    // direct loads address a tile's rows with 32-bit offsets from its first
    // row; stochastic rounding (bound by its Philox arithmetic) stays on the
    // register-fed kernel, whose tile also holds the column words.  Column
    // copies with a tensor scale take the direct-load kernel too: measured
    // 17% faster at 16384x14336, within 1% either way at 4096^2 to 8192^2.
    const bool dma = !SR && a.vec != 0 &&
                     (a.cols * SrcT<SRC>::bytes) % 16 == 0 &&
                     a.ld * SrcT<SRC>::bytes * 128 < (int64_t(1) << 32);
    const size_t dyn = SR ? (size_t)TR * TC * sizeof(uint32_t) : 0;
    const int tcols = dma ? DmaTile<SRC>::COLS : TC, trows = dma ? DmaTile<SRC>::ROWS : TR;
    a.ntx = (a.cols + tcols - 1) / tcols;
    a.ntiles = a.ntx * ((a.rows + trows - 1) / trows);
    const void* fn = dma ? reinterpret_cast<const void*>(&k_quant_tile_dma<SRC, FMT, ROW>)
                         : reinterpret_cast<const void*>(&k_quant_tile_reg<SRC, FMT, ROW, SR>);
    const int threads = dma ? 64 * (DmaTile<SRC>::NCW + 1) : 256;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, dyn);
    if (e != hipSuccess) return e;
    per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
    int64_t grid = (int64_t)cus * per_cu;
    grid = grid < a.ntiles ? grid : a.ntiles;
    if constexpr (!SR) {
        if (dma) {
            k_quant_tile_dma<SRC, FMT, ROW><<<dim3((unsigned)grid), dim3(threads), 0, stream>>>(a);
            return hipGetLastError();
        }
    }
    k_quant_tile_reg<SRC, FMT, ROW, SR><<<dim3((unsigned)grid), dim3(256), dyn, stream>>>(a);
    return hipGetLastError();
}

template <int SRC, int FMT>
hipError_t launch_fmt(const QuantJob& j, hipStream_t stream)
{
    QArgs a;
    a.x = j.x; a.rows = j.rows; a.cols = j.cols; a.ld = j.ld;
    a.q_row = j.q_row; a.s_row = j.s_row; a.q_col = j.q_col; a.s_col = j.s_col;
    a.tscale = j.tensor_scale;
    a.k0 = (uint32_t)j.seed; a.k1 = (uint32_t)(j.seed >> 32); a.offset = j.offset;
    a.hadamard = j.hadamard; a.two_level = j.two_level;
    const int es = j.src == SRC_BF16 ? 2 : 4;
    a.vec = ((reinterpret_cast<uintptr_t>(j.x) & 15u) == 0) && ((j.ld * es) % 16 == 0);
    a.ntx = a.ntiles = 0;                 // set by the tile launcher

    if (j.two_level == 1) {
        // partial keys parked in the scale array this call overwrites later
        uint8_t* sbuf = j.s_row ? j.s_row : j.s_col;
        const int64_t sbytes = j.s_row ? j.rows * (j.cols / 32) : j.cols * (j.rows / 32);
        const uintptr_t pad = (4 - (reinterpret_cast<uintptr_t>(sbuf) & 3u)) & 3u;
        const int64_t cap = (sbytes - (int64_t)pad) / 4;
        const int flat16 = a.vec && j.ld == j.cols;
        const int64_t nwords = j.rows * j.cols * es / 16;
        // at most 256 partials (one workgroup per CU): measured 0-3.5% faster
        // than 128 or 512-4096 at 4096^2 to 16384x14336
        int64_t want = flat16 ? (nwords + 4095) / 4096 : j.rows;
        want = want < 1 ? 1 : (want > 256 ? 256 : want);
        uint32_t* partial = (uint32_t*)(sbuf + pad);
        int64_t n = want < cap ? want : cap;
        if (n < 1) {                       // tiny tensor: the tensor-scale word holds the key
            n = 1;
            partial = (uint32_t*)j.tensor_scale;
        }
        k_amax_partial<SRC><<<dim3((unsigned)n), dim3(256), 0, stream>>>(j.x, j.rows, j.cols, j.ld, flat16, partial);
        k_amax_reduce<FMT><<<dim3(1), dim3(256), 0, stream>>>(partial, (int)n, j.tensor_scale);
    }
    if (j.q_col) {
        if (j.q_row) return j.sr ? launch_tile<SRC, FMT, true, true>(a, stream) : launch_tile<SRC, FMT, true, false>(a, stream);
        return j.sr ? launch_tile<SRC, FMT, false, true>(a, stream) : launch_tile<SRC, FMT, false, false>(a, stream);
    }
    const int64_t nblk = j.cols / 32;
    int64_t gy = (j.rows + 3) / 4;
    gy = gy > 65535 ? 65535 : gy;
    const dim3 grid((unsigned)((nblk + 63) / 64), (unsigned)gy);
    if (j.sr) k_quant_row<SRC, FMT, true><<<grid, dim3(256), 0, stream>>>(a);
    else k_quant_row<SRC, FMT, false><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

// partial maxima per tensor of the prediction (W's in work[0, 512), g's in
// work[512, 1024)): at most one workgroup per 2048 16-byte words
constexpr int kPredictPartials = 512;

template <int SRC, int FMT>
hipError_t launch_predict_t(const PredictJob& j, hipStream_t stream)
{
    constexpr int es = SrcT<SRC>::bytes;
    int n[2], flat[2];
    const void* src[2] = {j.w, j.g};
    const int64_t ld[2] = {j.ld_w, j.ld_g};
    for (int t = 0; t < 2; t++) {
        flat[t] = ((reinterpret_cast<uintptr_t>(src[t]) & 15u) == 0) && ld[t] == j.cols && (j.cols * es) % 16 == 0;
        const int64_t nwords = j.rows * j.cols * es / 16;
        int64_t want = flat[t] ? (nwords + 2047) / 2048 : j.rows;
        n[t] = (int)(want < 1 ? 1 : (want > kPredictPartials ? kPredictPartials : want));
    }
    k_amax_partial2<SRC><<<dim3((unsigned)(n[0] + n[1])), dim3(256), 0, stream>>>(
        j.w, j.ld_w, flat[0], j.work, n[0], j.g, j.ld_g, flat[1], j.work + kPredictPartials, j.rows, j.cols);
    k_predict_scale<FMT><<<dim3(1), dim3(256), 0, stream>>>(j.work, n[0], j.work + kPredictPartials, n[1], j.lr,
                                                            j.scale_out);
    return hipGetLastError();
}

// Scratch of the no-allocation prediction entry point: the partial maxima
// of W (words [0, 512)) and of g (words [512, 1024)), the same layout the
// caller's workspace has in mx_predict_tensor_scale.  Each GPU holds its
// own copy until the process ends; every call on that GPU shares it, so
// calls that overlap on one GPU race.  Nothing in it needs clearing: each
// call writes every partial word it then reads.
constexpr int kPredictScratchWords = 2 * kPredictPartials;
__device__ __align__(256) uint32_t scratch[kPredictScratchWords];

namespace {
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
uint32_t* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the device that owns `stream`, looked
// up once per device (with that device current) and kept: host code never
// passes the array's own name, which on the host is only a stand-in.
hipError_t scratch_on(hipStream_t stream, uint32_t** out)
{
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        g_scratch[dev] = (uint32_t*)p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_predict_noalloc(PredictJob j, hipStream_t stream)
{
    // the partial counts are capped at kPredictPartials per tensor
    // (launch_predict_t), so every input size fits the scratch words
    uint32_t* p = nullptr;
    const hipError_t e = scratch_on(stream, &p);
    if (e != hipSuccess) return e;
    j.work = p;
    return launch_predict(j, stream);
}

hipError_t launch_predict(const PredictJob& j, hipStream_t stream)
{
    const bool bf = j.src == SRC_BF16;
    switch (j.fmt) {
    case E4M3: return bf ? launch_predict_t<SRC_BF16, E4M3>(j, stream) : launch_predict_t<SRC_F32, E4M3>(j, stream);
    case E5M2: return bf ? launch_predict_t<SRC_BF16, E5M2>(j, stream) : launch_predict_t<SRC_F32, E5M2>(j, stream);
    default:   return bf ? launch_predict_t<SRC_BF16, E2M1>(j, stream) : launch_predict_t<SRC_F32, E2M1>(j, stream);
    }
}

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
