// mx_device.h -- device helpers for the gfx950 MX kernels: element-format
// traits, exact scaling, saturating round-to-nearest-even through the
// hardware FP8/FP4 converters, software stochastic rounding, Philox4x32-10,
// and the fixed-sign 32-point Hadamard butterfly.
//
// Sources (web pages; cited as [tag, section]):
//   [MOSS] "MOSS: 用微缩放和自动缩放实现无损 FP8 训练，OLMo-7B 加速 34%"
//   [FAF]  "格式感知融合:让FP4预训练提速两倍的工程实践"
//   Element encodings and the shared-exponent rule: OCP Microscaling (MX)
//   Formats specification v1.0.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef short short2v __attribute__((ext_vector_type(2)));

enum : int { E4M3 = 0, E5M2 = 1, E2M1 = 2 };
enum : int { SRC_F32 = 0, SRC_BF16 = 1 };

// Element-format traits.  emax: exponent of the largest finite value; emin:
// exponent of the smallest normal; mbits: stored mantissa bits; fmax: the
// largest finite value (E4M3 448, E5M2 57344, E2M1 6).
template <int FMT> struct Fmt;
template <> struct Fmt<E4M3> {
    static constexpr int bits = 8, emax = 8, emin = -6, mbits = 3;
    static constexpr float fmax = 448.0f;
};
template <> struct Fmt<E5M2> {
    static constexpr int bits = 8, emax = 15, emin = -14, mbits = 2;
    static constexpr float fmax = 57344.0f;
};
template <> struct Fmt<E2M1> {
    static constexpr int bits = 4, emax = 2, emin = 0, mbits = 1;
    static constexpr float fmax = 6.0f;
};

// 2^k as an fp32 for k in [-126, 127] (exact; built from the exponent field)
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// bf16 pair in one dword -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| bits as an unsigned key: ordered like |x| for finite values, Inf above
// every finite value and NaN above Inf.
__device__ __forceinline__ uint32_t abs_key(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// OCP shared exponent from the block's |max| key: floor(log2(amax)) - emax,
// clamped to [-127, 127]; -127 for an all-zero block.  Works on the fp32
// exponent field, so fp32 subnormal maxima get their true exponent.
template <int FMT>
__device__ __forceinline__ int block_exponent(uint32_t amax_key)
{
    // a zero or fp32-subnormal maximum (exponent <= -127) always clamps to -127
    const int ef = (int)(amax_key >> 23);
    if (ef == 0) return -127;
    int e = ef - 127 - Fmt<FMT>::emax;
    e = e < -127 ? -127 : e;
    return e;                      // <= 127 - emax for finite fp32 maxima
}

// v * 2^-e for a shared exponent of a finite block, e in [-127, 125]: one
// multiply by a normal fp32 power of two.  Exact unless the result falls
// below 2^-126, where every element format rounds it to a signed zero.
__device__ __forceinline__ float scale_by(float v, int e) { return v * exp2i(-e); }

// ---------------------------------------------------------------------
// Encoding of already-scaled values.  The gfx950 converters round to
// nearest-even exactly (including subnormal outputs and signed zero) but do
// not saturate, so the value is clamped to +-fmax first, which gives the
// saturating RNE of the OCP definition.
// ---------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ float clamp_fmax(float y)
{
    return __builtin_amdgcn_fmed3f(y, -Fmt<FMT>::fmax, Fmt<FMT>::fmax);
}

// four FP8 codes (y0 lowest byte ... y3 highest) in one dword: the converter
// writes a 16-bit half of its destination and keeps the other half.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4_fp8(float y0, float y1, float y2, float y3)
{
    if constexpr (FMT == E4M3) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, lo, true);
    } else {
        const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, lo, true);
    }
}

// eight FP4 codes in one dword (element 2j in the low nibble of byte j): the
// converter writes one byte of its destination and keeps the others.  The
// scale operand is 1.0, i.e. the values are already scaled.
__device__ __forceinline__ uint32_t cvt8_fp4(const float* y)
{
    uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, y[2], y[3], 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, y[4], y[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, y[6], y[7], 1.0f, 3);
}

// ---------------------------------------------------------------------
// Stochastic rounding ([FAF, "两个关键的数值技巧"]): with lo <= |y| < hi the
// neighbouring representable magnitudes and F = floor((|y|-lo)/(hi-lo) *
// 2^32), round up iff u < F.  Returns the chosen value (exactly
// representable, sign of y kept); |y| >= fmax saturates.
// ---------------------------------------------------------------------
//
// Computed in fixed point from the bits of |y|: with m the biased exponent
// of the quantum's binade (that of |y|, at least the format's emin), |y| /
// quantum = 24-bit significand x 2^-(23 - mbits + (m - e)); placing the
// significand at bit 32 of a 64-bit word and shifting it right by that
// amount (at most 63: smaller values have no bits at or above 2^-32) leaves
// floor(|y| / quantum) in the high word and F in the low one.  The lower
// neighbour is then that integer times the quantum, the upper one the next
// multiple, and a value at or above fmax gives at least fmax on both sides.
// This yields the definition's F and neighbours for every finite fp32 value
// in all three formats.
template <int FMT>
__device__ __forceinline__ float sr_value(float y, uint32_t u)
{
    constexpr int MB = Fmt<FMT>::mbits, EMINB = Fmt<FMT>::emin + 127;
    const uint32_t ab = __float_as_uint(y) & 0x7FFFFFFFu;
    const int eb = (int)(ab >> 23);                         // 0 for zero and fp32 subnormals
    const int m = eb > EMINB ? eb : EMINB;
    const int rs = min(23 - MB + (m - eb), 63);
    const uint64_t X = ((uint64_t)((ab & 0x007FFFFFu) | 0x00800000u) << 32) >> rs;
    const uint32_t n = (uint32_t)(X >> 32) + ((u < (uint32_t)X) ? 1u : 0u);
    const float r = fminf(ldexpf((float)n, m - 127 - MB), Fmt<FMT>::fmax);
    return __builtin_copysignf(r, y);
}

// ---------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11)
// ---------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; r++) {
        // one 32x32->64 product gives both halves (a single v_mad_u64_u32)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        // (three-input XORs: one v_bitop3_b32 each, truth table 0x96)
        c = u32x4{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                  (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Random word for the element with row-major source index idx: counter
// (idx>>2 low, idx>>2 high, axis, offset), key (seed low, seed high), word idx&3.
__device__ __forceinline__ u32x4 philox_block(uint64_t n, uint32_t axis, uint32_t offset,
                                              uint32_t k0, uint32_t k1)
{
    return philox4x32_10(u32x4{(uint32_t)n, (uint32_t)(n >> 32), axis, offset}, k0, k1);
}

__device__ __forceinline__ uint32_t pick(const u32x4& w, uint32_t i)
{
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// ---------------------------------------------------------------------
// Fixed-sign 32-point Hadamard ([FAF, "两个关键的数值技巧"]): Sylvester
// order, unnormalised, stages h = 1, 2, 4, 8, 16; at each stage the pair
// (a, b) = (v[i], v[i+h]) becomes (a+b, a-b) in fp32.
// ---------------------------------------------------------------------
__device__ __forceinline__ void fwht32(float* v)
{
#pragma unroll
    for (int st = 0; st < 5; st++) {
        const int h = 1 << st;
#pragma unroll
        for (int i = 0; i < 32; i++)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    }
}

// fwht32 that also returns the |max| key of its output.  Of the last
// stage's pair, max(|RN(a+b)|, |RN(a-b)|) = RN(|a|+|b|): one of the two is
// the sum of the magnitudes and the other their difference, and rounding to
// nearest is monotone and odd-symmetric.  So 16 sums of magnitudes give the
// key instead of 32 abs-max steps.  A block holding a NaN or an Inf, or
// whose transform overflows, gets a key of at least 0x7F800000 either way
// (Inf - Inf gives an Inf key here where the output holds a NaN).
__device__ __forceinline__ uint32_t fwht32_key(float* v)
{
#pragma unroll
    for (int st = 0; st < 4; st++) {
        const int h = 1 << st;
#pragma unroll
        for (int i = 0; i < 32; i++)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    }
    uint32_t key = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float a = v[i], b = v[i + 16];
        v[i] = a + b;
        v[i + 16] = a - b;
        // the sums are +0 or more, or NaN: the largest raw pattern,
        // its sign cleared, is the key
        key = max(key, __float_as_uint(fabsf(a) + fabsf(b)));
    }
    return key & 0x7FFFFFFFu;
}

// ---------------------------------------------------------------------------
// x / s_t rounded to nearest even, with the divisor s_t shared by many
// quotients (a tensor scale, a group maximum).  The
// reciprocal r = RN(1/s_t) is formed once; q = RN(x r) refined by one exact
// residual step q' = RN(q + RN(x - q s_t) r) equals the IEEE quotient.  This
// is Markstein's correction theorem (P. Markstein, IBM J. Res. Dev. 34(1),
// 1990; Theorem 8.10 of Muller et al., Handbook of Floating-Point
// Arithmetic): if r is within half an ulp of 1/s_t (here r = RN(1/s_t))
// and q within one ulp of x/s_t (q = RN(x r) is: the reciprocal's half-ulp
// error and the product's rounding stay below one ulp), the residual
// x - q s_t is exactly representable and one FMA returns RN(x/s_t) --
// provided nothing underflows or overflows along the way.  The range checks
// keep away from those cases: the kernels require |x|, |q'| >= 2^-96 and
// |q'| <= 2^17 (the range over which the identity was also checked
// exhaustively, every fp32 x against divisors with adversarial
// significands).  Per block they check |x| >= T = max(2^-96, 2^-95 |s_t|)
// for every nonzero x (which implies |q'| >= 2^-96) and |q'| <= 2^17 on the
// block's largest quotient; a block that fails takes the IEEE division.
// Zeros keep the sign of x r; a non-finite x makes the block non-finite
// either way.
struct TensorDiv {
    float s, r;
    uint32_t lo_key;    // (bits(T) << 1) - 1
    bool fast;          // s and 1/s are normal fp32 numbers
};

__device__ __forceinline__ TensorDiv make_div(float s)
{
    TensorDiv d;
    const float as = fabsf(s);
    d.s = s;
    d.r = 1.0f / s;
    d.fast = as > 0x1p-125f && as < 0x1p125f;
    const float t = d.fast ? fmaxf(0x1p-96f, 0x1p-95f * as) : 1.0f;
    d.lo_key = (__float_as_uint(t) << 1) - 1u;
    return d;
}

// fast quotient; `lo` tracks min((bits(x) << 1) - 1), whose value is below
// lo_key exactly when some nonzero |x| < T
__device__ __forceinline__ float div_fast(float x, const TensorDiv& d, uint32_t& lo)
{
    const float q0 = x * d.r;
    const float rem = __builtin_fmaf(-q0, d.s, x);
    const float q1 = __builtin_fmaf(rem, d.r, q0);
    lo = min(lo, (__float_as_uint(x) << 1) - 1u);
    return __builtin_copysignf(q1, q0);
}

}  // namespace mx
