// optstate.hip -- FP8 optimizer states with dynamic range expansion.
//
// [COAT, "解決方案：動態範圍擴充套件"]: before an optimizer state (Adam's first
// or second moment) is quantized to FP8, an expansion function with one
// parameter k per quantization group, computed on the fly, stretches the
// group's max/min ratio to the format's own (about 2e5 for E4M3), so that
// the group uses the whole span from the smallest subnormal to the largest
// value instead of a sliver of it.  The page lost the formula; this follows
// the COAT paper it cites: f(x) = sign(x) |x|^k.  Per group of G values:
//   amax = max |x|,  amin = min nonzero |x|,
//   k    = log2(Fmax / smallest subnormal) / log2(amax / amin)  (1 if amax == amin),
//   code = RNE_sat( sign(x) * (|x| / amax)^k * Fmax ),
// so the group's largest magnitude maps to Fmax and its smallest nonzero
// one to the smallest subnormal.  amax and k are stored per group; the
// inverse is x = sign(code) * amax * (|decode(code)| / Fmax)^(1/k).
// (Normalising by amax keeps every power inside fp32 range; the paper's
// per-group scale of f(x) is then amax^k / Fmax, implicit.)
//
// The powers are exp2(k log2 u) with log2 and exp2 evaluated as a fixed
// sequence of fp32 operations -- log2 as e + z P(z) with z = m - 1 on the
// reduced mantissa m in (sqrt(1/2), sqrt(2)), exp2 as 2^n Q(y - n) with n
// the nearest integer, P and Q polynomial fits evaluated by fused
// multiply-adds -- each operation rounded once, in the order written
// (contraction off), so that the codes are a plain function of IEEE fp32
// arithmetic rather than of a hardware transcendental's approximation.
// Accuracy: a few fp32 ulps for log2 and exp2, about 1e-6 relative for the
// powers, far below an FP8 step.
//
// 4 bytes read and 1 written per element, 8 bytes of parameters per group;
// the exact fp32 sequence makes the kernels bound by VALU work, so both
// kernels are written to spend as few instructions per element as the
// arithmetic allows while computing the same bits:
//  - log2 splits x into m and e with one integer subtraction of the bits of
//    sqrt(1/2) (the exponent field drops by one exactly when the mantissa
//    lies above sqrt(2)), and exp2 takes its special cases as selects, so
//    that neither has a branch;
//  - one thread handles 16 elements (four 16-byte loads, each contiguous
//    across the threads of a group), so that the per-group work (the
//    reductions, k, the reciprocal of amax) is shared by more elements;
//  - the quantizer's |x|/amax uses the reciprocal-plus-residual division
//    (TensorDiv: the IEEE quotient) when the group's smallest nonzero
//    magnitude is above the division's threshold; then every quotient is
//    normal and log2 needs no subnormal step.  Otherwise the group takes the
//    IEEE division and the general log2;
//  - the dequantizer looks log2 of each decoded magnitude up in a
//    per-workgroup table, since it depends on the code alone.
#include <type_traits>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

namespace {

// log2 of the format's dynamic range Fmax / smallest subnormal, rounded to
// fp32: E4M3 448 / 2^-9 = 2^17.807..., E5M2 57344 / 2^-16 = 2^31.807...
template <int FMT> struct Range;
template <> struct Range<E4M3> { static constexpr float log2r = 17.8073549f; };
template <> struct Range<E5M2> { static constexpr float log2r = 31.8073549f; };

// log2 from the bits of a normal x > 0 (or +Inf), less `sub`: x = m * 2^e
// with m in (sqrt(1/2), sqrt(2)), z = m - 1 (exact), log2 x = e + z * P(z),
// P of degree 8 (a least-squares fit of log2(1+z)/z on that range,
// coefficients rounded to fp32), every step one fused multiply-add, in the
// order written.  Subtracting the bits of the smallest fp32 above sqrt(1/2)
// borrows from the exponent field exactly when the mantissa is at most
// sqrt(2), so the arithmetic shift gives e and the low 23 bits, added back,
// give m.
__device__ __forceinline__ float log2_bits(uint32_t bits, int sub)
{
#pragma clang fp contract(off)
    const uint32_t d = bits - 0x3F3504F4u;
    const int ex = ((int32_t)d >> 23) - sub;
    const float z = __uint_as_float((d & 0x007FFFFFu) + 0x3F3504F4u) - 1.0f;   // exact
    float p = 0x1.025a88p-3f;
    p = __builtin_fmaf(p, z, -0x1.a8cd06p-3f);
    p = __builtin_fmaf(p, z, 0x1.b9b144p-3f);
    p = __builtin_fmaf(p, z, -0x1.e94efep-3f);
    p = __builtin_fmaf(p, z, 0x1.26d40cp-2f);
    p = __builtin_fmaf(p, z, -0x1.715c9cp-2f);
    p = __builtin_fmaf(p, z, 0x1.ec73d4p-2f);
    p = __builtin_fmaf(p, z, -0x1.71547p-1f);
    p = __builtin_fmaf(p, z, 0x1.715476p+0f);
    return __builtin_fmaf(z, p, (float)ex);
}

// log2 of x >= 2^-126 (or +Inf)
__device__ __forceinline__ float log2_normal(float x) { return log2_bits(__float_as_uint(x), 0); }

// log2 of x > 0 (finite or +Inf): a subnormal x is first scaled into the
// normal range (exact)
__device__ __forceinline__ float log2_fixed(float x)
{
#pragma clang fp contract(off)
    const bool sub = x < 0x1p-126f;
    return log2_bits(__float_as_uint(sub ? x * 0x1p32f : x), sub ? 32 : 0);
}

// 2^y for y in [-151, 128]: n = floor(y + 1/2), z = y - n (exact, |z| <=
// 1/2), 2^z from a degree-6 fit on [-1/2, 1/2] whose constant term is
// exactly 1, then 2^n
__device__ __forceinline__ float exp2_core(float y)
{
#pragma clang fp contract(off)
    const float n = floorf(y + 0.5f);
    const float z = y - n;
    float s = 0x1.41a7p-13f;
    s = __builtin_fmaf(s, z, 0x1.5f44f4p-10f);
    s = __builtin_fmaf(s, z, 0x1.3b2dfep-7f);
    s = __builtin_fmaf(s, z, 0x1.c6aed6p-5f);
    s = __builtin_fmaf(s, z, 0x1.ebfbdap-3f);
    s = __builtin_fmaf(s, z, 0x1.62e43p-1f);
    s = __builtin_fmaf(s, z, 1.0f);
    return ldexpf(s, (int)n);
}

// 2^y for y <= 0, not NaN: 0 below -150
__device__ __forceinline__ float exp2_nonpos(float y)
{
    const float r = exp2_core(fmaxf(y, -151.0f));
    return y < -150.0f ? 0.0f : r;
}

// 2^y for any y: NaN for NaN, +Inf from 128 up, 0 below -150
__device__ __forceinline__ float exp2_fixed(float y)
{
    const float r = exp2_core(fminf(fmaxf(y, -151.0f), 128.0f));
    const float o = y < -150.0f ? 0.0f : y >= 128.0f ? __builtin_inff() : r;
    return y != y ? y : o;
}

// u^k for u >= 0
__device__ __forceinline__ float pow_fixed(float u, float k)
{
#pragma clang fp contract(off)
    const float p = exp2_fixed(k * log2_fixed(u));
    return u == 0.0f ? 0.0f : p;
}

// exact fp32 value of an FP8 code
template <int FMT>
__device__ __forceinline__ float decode8(uint32_t c)
{
    constexpr int MB = Fmt<FMT>::mbits, EB = 7 - MB, BIAS = FMT == E4M3 ? 7 : 15;
    const uint32_t e = (c >> MB) & ((1u << EB) - 1u), m = c & ((1u << MB) - 1u);
    float v;
    if (FMT == E4M3 && e == 15 && m == 7) v = __builtin_nanf("");
    else if (FMT == E5M2 && e == 31) v = m ? __builtin_nanf("") : __builtin_inff();
    else if (e == 0) v = (float)m * exp2i(1 - BIAS - MB);
    else v = (float)((1u << MB) | m) * exp2i((int)e - BIAS - MB);
    return (c & 0x80u) ? -v : v;
}

// Both kernels: T = G / (4 NV) threads per group, thread j of group g
// handles the float4 (and code word) offsets j, j + T, ..., j + (NV-1) T of
// the group, so that each of its NV loads and stores is contiguous across
// the group's threads.
template <int FMT, int G, int NV>
__global__ __launch_bounds__(256) void k_optstate_quant(const float4* __restrict__ x, int64_t ngroups,
                                                        uint32_t* __restrict__ q, float* __restrict__ gamax,
                                                        float* __restrict__ gk)
{
#pragma clang fp contract(off)
    constexpr int T = G / (4 * NV), E = 4 * NV;
    static_assert(T >= 1 && T <= 64 && (T & (T - 1)) == 0, "a group's threads lie inside one wave");
    const int64_t nthreads = ngroups * T;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t - (threadIdx.x & 63) < nthreads;
         t += (int64_t)gridDim.x * 256) {
        // every lane of a wave stays in the loop while any lane of the wave has
        // work, so the group shuffles below see all their lanes
        const bool live = t < nthreads;
        const int64_t g = t / T;
        const int j = (int)(t & (T - 1));
        const int64_t base = g * (G / 4) + j;
        float xs[E], a[E];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const float4 v = live ? x[base + i * T] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            xs[4 * i] = v.x; xs[4 * i + 1] = v.y; xs[4 * i + 2] = v.z; xs[4 * i + 3] = v.w;
        }
        // group maximum and smallest nonzero magnitude as integer extrema of
        // |x|'s bits (their order is the values' for finite magnitudes; Inf
        // and NaN bits lie above every finite one, so they flag the group by
        // themselves).  The minimum runs over bits - 1, which sends zeros to
        // the top of the unsigned range.
        uint32_t kmax = 0, kmin = ~0u;
#pragma unroll
        for (int e = 0; e < E; e++) {
            const uint32_t b = __float_as_uint(xs[e]) & 0x7FFFFFFFu;
            a[e] = __uint_as_float(b);
            kmax = max(kmax, b);
            kmin = min(kmin, b - 1u);
        }
        // butterflies inside 32-lane halves by swizzle (xor mask in bits 14:10,
        // and mask 0x1F), across halves by a permute
        auto step = [&](auto OFFC) __attribute__((always_inline)) {
            constexpr int off = decltype(OFFC)::value;
            if constexpr (off < T && off < 32) {
                kmax = max(kmax, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kmax, 0x1F | (off << 10)));
                kmin = min(kmin, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kmin, 0x1F | (off << 10)));
            } else if constexpr (off < T) {
                kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
                kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
            }
        };
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 8>{});
        step(std::integral_constant<int, 16>{});
        step(std::integral_constant<int, 32>{});
        const float amin = __uint_as_float(kmin + 1u);  // used only when some |x| > 0
        const bool bad = kmax >= 0x7F800000u;
        const float amax = __uint_as_float(kmax);
        if (!live) continue;
        const bool lead = j == 0;
        uint32_t codes[NV];
        if (bad) {                                   // a NaN or Inf: the NaN code everywhere
#pragma unroll
            for (int i = 0; i < NV; i++) codes[i] = 0x7F7F7F7Fu;
            if (lead) { gamax[g] = __builtin_nanf(""); gk[g] = __builtin_nanf(""); }
        } else if (amax == 0.0f) {                   // all zero: signed zeros, unit parameters
#pragma unroll
            for (int i = 0; i < NV; i++)
                codes[i] = (__float_as_uint(xs[4 * i]) >> 31) << 7 | (__float_as_uint(xs[4 * i + 1]) >> 31) << 15 |
                           (__float_as_uint(xs[4 * i + 2]) >> 31) << 23 | (__float_as_uint(xs[4 * i + 3]) >> 31) << 31;
            if (lead) { gamax[g] = 1.0f; gk[g] = 1.0f; }
        } else {
            const float r = amax / amin;             // >= 1: normal or +Inf
            const float k = r > 1.0f ? Range<FMT>::log2r / log2_normal(r) : 1.0f;
            // k is finite and positive, and every quotient u = |x|/amax lies in
            // [0, 1], so y = k log2 u is finite and at most 0 for u > 0
            float y[E];
            const TensorDiv d = make_div(amax);
            if (d.fast && ((kmin + 1u) << 1) - 1u >= d.lo_key) {
                // every nonzero |x| of the group is at least amin, at or above the
                // division's threshold: the fast form gives the IEEE quotient
                // (+0 for x = 0, a normal number otherwise), and log2 needs no
                // subnormal step.  Two steps of the general form are left out
                // because they cannot change a code: 2^y is at most 1 for y <= 0,
                // so |x|'s value stays within Fmax without the clamp; and below
                // y = -150, where the general form returns 0, the power is at most
                // 2^-149 and its product with Fmax far below the format's smallest
                // subnormal, so it rounds to a zero code (of x's sign) just as 0
                // does.
#pragma unroll
                for (int e = 0; e < E; e++) {
                    const float q0 = a[e] * d.r;
                    const float u = __builtin_fmaf(__builtin_fmaf(-q0, d.s, a[e]), d.r, q0);
                    const float p = exp2_core(fmaxf(k * log2_normal(u), -151.0f));
                    y[e] = __builtin_copysignf((u == 0.0f ? 0.0f : p) * Fmt<FMT>::fmax, xs[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; e++)
                    y[e] = clamp_fmax<FMT>(__builtin_copysignf(pow_fixed(a[e] / amax, k) * Fmt<FMT>::fmax, xs[e]));
            }
#pragma unroll
            for (int i = 0; i < NV; i++) codes[i] = cvt4_fp8<FMT>(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
            if (lead) { gamax[g] = amax; gk[g] = k; }
        }
#pragma unroll
        for (int i = 0; i < NV; i++) q[base + i * T] = codes[i];
    }
}

template <int FMT, int G, int NV>
__global__ __launch_bounds__(256) void k_optstate_dequant(const uint32_t* __restrict__ q, const float* __restrict__ gamax,
                                                          const float* __restrict__ gk, int64_t ngroups,
                                                          float4* __restrict__ out)
{
#pragma clang fp contract(off)
    constexpr int T = G / (4 * NV);
    static_assert(T >= 1 && (T & (T - 1)) == 0, "threads per group");
    // NaN codes: E4M3 0x7F; E5M2 0x7D-0x7F (0x7C is Inf)
    auto is_nan = [](uint32_t c7) { return FMT == E4M3 ? c7 == 0x7Fu : c7 > 0x7Cu; };
    // log2(|decode(c)| / Fmax) for the 128 magnitudes, in the same fixed
    // sequence the per-element form evaluates; -Inf for code 0 (so that its
    // power is 0 whenever the exponent 1/k is positive) and 0 for the NaN
    // codes, whose output is NaN whatever the power
    __shared__ float lg[128];
    for (int c = threadIdx.x; c < 128; c += 256)
        lg[c] = c == 0 ? -__builtin_inff()
                       : is_nan((uint32_t)c) ? 0.0f : log2_fixed(fabsf(decode8<FMT>((uint32_t)c)) / Fmt<FMT>::fmax);
    __syncthreads();
    const int64_t nthreads = ngroups * T;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < nthreads; t += (int64_t)gridDim.x * 256) {
        const int64_t g = t / T;
        const int64_t base = g * (G / 4) + (t & (T - 1));
        uint32_t c4[NV];
#pragma unroll
        for (int i = 0; i < NV; i++) c4[i] = q[base + i * T];
        const float amax = gamax[g], k = gk[g];
        const float kinv = 1.0f / k;
        const bool nan_group = amax != amax || k != k;
        // the table reads first, then arithmetic without branches; a NaN
        // output comes from adding NaN (others add -0, which changes nothing)
        float l[4 * NV], o[4 * NV];
#pragma unroll
        for (int e = 0; e < 4 * NV; e++) l[e] = lg[(c4[e / 4] >> (8 * (e % 4))) & 0x7Fu];
        auto run = [&](auto SIMPLE) __attribute__((always_inline)) {
#pragma clang fp contract(off)
#pragma unroll
            for (int e = 0; e < 4 * NV; e++) {
                const uint32_t c = (c4[e / 4] >> (8 * (e % 4))) & 0xFFu, c7 = c & 0x7Fu;
                const float y = kinv * l[e];
                float p;
                if constexpr (decltype(SIMPLE)::value) p = exp2_nonpos(y);    // 0 for code 0 (y = -Inf)
                else p = c7 == 0 ? 0.0f : exp2_fixed(y);
                const float m = amax * p + (is_nan(c7) || nan_group ? __builtin_nanf("") : -0.0f);
                o[e] = (c & 0x80u) ? -m : m;
            }
        };
        // E4M3 has no Inf code, so every non-NaN code has lg <= 0; with
        // 0 < kinv < Inf every y is then at most 0 and not NaN
        if (FMT == E4M3 && kinv > 0.0f && kinv < __builtin_inff()) run(std::true_type{});
        else run(std::false_type{});
#pragma unroll
        for (int i = 0; i < NV; i++) out[base + i * T] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
}

// enough workgroups to cover the elements, at most 16 per CU (grid-stride loops)
unsigned grid_for(int64_t nthreads)
{
    int64_t wg = (nthreads + 255) / 256;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t cap = (int64_t)cus * 16;
    return (unsigned)(wg < cap ? (wg < 1 ? 1 : wg) : cap);
}

template <int FMT, int G>
hipError_t launch_os(const OptStateJob& j, hipStream_t s)
{
    // float4 per thread: 4 measured fastest for the quantizer (2 and 8 both
    // about 5% slower on 117M elements)
    constexpr int NV = 4;
    const int64_t ngroups = j.n / G, nthreads = ngroups * (G / (4 * NV));
    if (j.dequant)
        k_optstate_dequant<FMT, G, NV><<<grid_for(nthreads), 256, 0, s>>>((const uint32_t*)j.q, j.amax, j.k, ngroups,
                                                                         (float4*)j.out);
    else
        k_optstate_quant<FMT, G, NV><<<grid_for(nthreads), 256, 0, s>>>((const float4*)j.x, ngroups, (uint32_t*)j.q,
                                                                       j.amax, j.k);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_os_fmt(const OptStateJob& j, hipStream_t s)
{
    switch (j.group) {
    case 32: return launch_os<FMT, 32>(j, s);
    case 64: return launch_os<FMT, 64>(j, s);
    case 128: return launch_os<FMT, 128>(j, s);
    default: return launch_os<FMT, 256>(j, s);
    }
}

}  // namespace

hipError_t launch_optstate(const OptStateJob& j, hipStream_t stream)
{
    return j.fmt == E4M3 ? launch_os_fmt<E4M3>(j, stream) : launch_os_fmt<E5M2>(j, stream);
}

}  // namespace mx
