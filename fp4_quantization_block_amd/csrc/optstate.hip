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
// sequence of fp32 operations -- log2 from the atanh series in
// t = (m - 1)/(m + 1) on m in [sqrt(1/2), sqrt(2)), exp2 from the Taylor
// series of e^z, z = f ln 2, |f| <= 1/2 -- each operation rounded once, in
// the order written (contraction off), so that the codes are a plain
// function of IEEE fp32 arithmetic rather than of a hardware
// transcendental's approximation.  Accuracy: a few fp32 ulps for log2 and
// exp2, about 1e-6 relative for the powers, far below an FP8 step.
//
// 4 bytes read and 1 written per element, 8 bytes of parameters per group;
// the exact fp32 sequence makes the kernels bound by VALU work.  Two ways of
// doing less of it while computing the same bits: the quantizer's |x|/amax
// uses the reciprocal-plus-residual division (TensorDiv: the IEEE quotient,
// with the IEEE division as fallback), and the dequantizer looks log2 of
// each decoded magnitude up in a per-workgroup table, since it depends on
// the code alone.  One thread handles 4 consecutive elements (16-byte loads,
// 4-byte code stores); the G/4 threads of a group reduce amax and amin with
// lane shuffles inside their wave.
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

// log2 of x > 0 (finite or +Inf): x = m * 2^e with m in [sqrt(1/2),
// sqrt(2)), z = m - 1 (exact), log2 x = e + z * P(z), P of degree 8 (a
// least-squares fit of log2(1+z)/z on that range, coefficients rounded to
// fp32), every step one fused multiply-add, in the order written
__device__ __forceinline__ float log2_fixed(float x)
{
#pragma clang fp contract(off)
    int ex = 0;
    if (x < 0x1p-126f) {             // subnormal: scale into the normal range (exact)
        x = x * 0x1p32f;
        ex = -32;
    }
    const uint32_t bits = __float_as_uint(x);
    ex += (int)(bits >> 23) - 127;
    float m = __uint_as_float((bits & 0x007FFFFFu) | 0x3F800000u);     // [1, 2)
    if (m > 1.41421356f) {
        m = m * 0.5f;
        ex += 1;
    }
    const float z = m - 1.0f;                        // exact
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

// 2^y: y = n + z with n = floor(y + 1/2), z = y - n (exact), 2^z from a
// degree-6 fit on [-1/2, 1/2] whose constant term is exactly 1, then 2^n
__device__ __forceinline__ float exp2_fixed(float y)
{
#pragma clang fp contract(off)
    if (y != y) return y;
    if (y >= 128.0f) return __builtin_inff();
    if (y < -150.0f) return 0.0f;
    const float n = floorf(y + 0.5f);
    const float z = y - n;                           // exact, |z| <= 1/2
    float s = 0x1.41a7p-13f;
    s = __builtin_fmaf(s, z, 0x1.5f44f4p-10f);
    s = __builtin_fmaf(s, z, 0x1.3b2dfep-7f);
    s = __builtin_fmaf(s, z, 0x1.c6aed6p-5f);
    s = __builtin_fmaf(s, z, 0x1.ebfbdap-3f);
    s = __builtin_fmaf(s, z, 0x1.62e43p-1f);
    s = __builtin_fmaf(s, z, 1.0f);
    return ldexpf(s, (int)n);
}

// u^k for u >= 0
__device__ __forceinline__ float pow_fixed(float u, float k)
{
#pragma clang fp contract(off)
    if (u == 0.0f) return 0.0f;
    return exp2_fixed(k * log2_fixed(u));
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

template <int FMT, int G>
__global__ __launch_bounds__(256) void k_optstate_quant(const float4* __restrict__ x, int64_t ngroups,
                                                        uint32_t* __restrict__ q, float* __restrict__ gamax,
                                                        float* __restrict__ gk)
{
#pragma clang fp contract(off)
    constexpr int T = G / 4;                         // threads per group (8..64, inside one wave)
    const int64_t nthreads = ngroups * T;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t - (threadIdx.x & 63) < nthreads;
         t += (int64_t)gridDim.x * 256) {
        // every lane of a wave stays in the loop while any lane of the wave has
        // work, so the group shuffles below see all their lanes
        const bool live = t < nthreads;
        const float4 v = live ? x[t] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float a[4] = {fabsf(v.x), fabsf(v.y), fabsf(v.z), fabsf(v.w)};
        // group maximum as an integer maximum of |x|'s bits (the order of the
        // values for finite magnitudes; Inf and NaN bits lie above every
        // finite one, so they flag the group by themselves), and the
        // smallest nonzero magnitude
        uint32_t kmax = 0;
        float amin = __builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; i++) {
            kmax = max(kmax, __float_as_uint(a[i]));
            if (a[i] > 0.0f) amin = fminf(amin, a[i]);
        }
        // butterflies inside 32-lane halves by swizzle (xor mask in bits 14:10,
        // and mask 0x1F), across halves by a permute
        auto step = [&](auto OFFC) __attribute__((always_inline)) {
            constexpr int off = decltype(OFFC)::value;
            if constexpr (off < T && off < 32) {
                kmax = max(kmax, (uint32_t)__builtin_amdgcn_ds_swizzle((int)kmax, 0x1F | (off << 10)));
                amin = fminf(amin, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(amin), 0x1F | (off << 10))));
            } else if constexpr (off < T) {
                kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
                amin = fminf(amin, __shfl_xor(amin, off));
            }
        };
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 4>{});
        step(std::integral_constant<int, 8>{});
        step(std::integral_constant<int, 16>{});
        step(std::integral_constant<int, 32>{});
        const bool bad = kmax >= 0x7F800000u;
        const float amax = __uint_as_float(kmax);
        if (!live) continue;
        const int64_t g = t / T;
        const bool lead = (t % T) == 0;
        uint32_t codes;
        if (bad) {                                   // a NaN or Inf: the NaN code everywhere
            codes = 0x7F7F7F7Fu;
            if (lead) { gamax[g] = __builtin_nanf(""); gk[g] = __builtin_nanf(""); }
        } else if (amax == 0.0f) {                   // all zero: signed zeros, unit parameters
            codes = (__float_as_uint(v.x) >> 31) << 7 | (__float_as_uint(v.y) >> 31) << 15 |
                    (__float_as_uint(v.z) >> 31) << 23 | (__float_as_uint(v.w) >> 31) << 31;
            if (lead) { gamax[g] = 1.0f; gk[g] = 1.0f; }
        } else {
            const float r = amax / amin;
            const float k = r > 1.0f ? Range<FMT>::log2r / log2_fixed(r) : 1.0f;
            const float xs[4] = {v.x, v.y, v.z, v.w};
            // u = |x| / amax, the IEEE quotient (quotients are at most 1; an
            // element far below amax takes the IEEE division)
            const TensorDiv d = make_div(amax);
            uint32_t lo = ~0u;
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; i++) u[i] = div_fast(a[i], d, lo);
            if (!d.fast || lo < d.lo_key) {
#pragma unroll
                for (int i = 0; i < 4; i++) u[i] = a[i] / amax;
            }
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float e = pow_fixed(u[i], k) * Fmt<FMT>::fmax;
                y[i] = clamp_fmax<FMT>(__builtin_copysignf(e, xs[i]));
            }
            codes = cvt4_fp8<FMT>(y[0], y[1], y[2], y[3]);
            if (lead) { gamax[g] = amax; gk[g] = k; }
        }
        q[t] = codes;
    }
}

template <int FMT, int G>
__global__ __launch_bounds__(256) void k_optstate_dequant(const uint32_t* __restrict__ q, const float* __restrict__ gamax,
                                                          const float* __restrict__ gk, int64_t nthreads,
                                                          float4* __restrict__ out)
{
#pragma clang fp contract(off)
    constexpr int T = G / 4;
    // log2(|decode(c)| / Fmax) for the 128 magnitudes, in the same fixed
    // sequence the per-element form evaluates (code 0, whose power is 0, is
    // never looked up)
    __shared__ float lg[128];
    for (int c = threadIdx.x; c < 128; c += 256) lg[c] = log2_fixed(fabsf(decode8<FMT>((uint32_t)c)) / Fmt<FMT>::fmax);
    __syncthreads();
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < nthreads; t += (int64_t)gridDim.x * 256) {
        const uint32_t c4 = q[t];
        const int64_t g = t / T;
        const float amax = gamax[g], k = gk[g];
        const float kinv = 1.0f / k;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t c = (c4 >> (8 * i)) & 0xFFu, c7 = c & 0x7Fu;
            // NaN codes: E4M3 0x7F; E5M2 0x7D-0x7F (0x7C is Inf)
            const bool nan_code = FMT == E4M3 ? c7 == 0x7Fu : c7 > 0x7Cu;
            const float pw = c7 == 0 ? 0.0f : exp2_fixed(kinv * lg[c7]);
            float m = amax * pw;
            if (nan_code || amax != amax || k != k) m = __builtin_nanf("");
            o[i] = (c & 0x80u) ? -m : m;
        }
        out[t] = make_float4(o[0], o[1], o[2], o[3]);
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
    const int64_t ngroups = j.n / G, nthreads = j.n / 4;
    if (j.dequant)
        k_optstate_dequant<FMT, G><<<grid_for(nthreads), 256, 0, s>>>((const uint32_t*)j.q, j.amax, j.k, nthreads,
                                                                     (float4*)j.out);
    else
        k_optstate_quant<FMT, G><<<grid_for(nthreads), 256, 0, s>>>((const float4*)j.x, ngroups, (uint32_t*)j.q,
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
