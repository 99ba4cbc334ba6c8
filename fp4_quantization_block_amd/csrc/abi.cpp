// abi.cpp -- the C ABI of libmx.so (declared in include/mx.h).  Every entry
// point validates its arguments on the host before touching HIP; on an
// error it enqueues nothing and returns a status.  Nothing is allocated and
// no state is kept between calls (apart from a thread-local error text).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "../../include/mx.h"
#include "mx_internal.h"

namespace {

thread_local char g_msg[256] = "";

mx_status fail(mx_status s, const char* what)
{
    std::snprintf(g_msg, sizeof g_msg, "%s", what);
    return s;
}

mx_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return MX_OK;
    std::snprintf(g_msg, sizeof g_msg, "HIP: %s", hipGetErrorString(e));
    return MX_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_fmt(int32_t f) { return f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M1; }
int elem_bits(int32_t f) { return f == MX_E2M1 ? 4 : 8; }

mx_status check_cfg(const mx_qconfig* cfg, const float* tensor_scale)
{
    if (!cfg) return fail(MX_ERR_INVALID_ARG, "cfg is NULL");
    if (!valid_fmt(cfg->fmt)) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (cfg->block != 32) return fail(MX_ERR_INVALID_ARG, "block size must be 32");
    if (cfg->scale_fmt != MX_SCALE_E8M0 && cfg->scale_fmt != MX_SCALE_E8M0_TENSOR_F32)
        return fail(MX_ERR_INVALID_ARG, "unknown scale format");
    if (cfg->tscale != MX_TSCALE_COMPUTE && cfg->tscale != MX_TSCALE_PROVIDED)
        return fail(MX_ERR_INVALID_ARG, "unknown tensor-scale mode");
    if (cfg->rounding != MX_RNE && cfg->rounding != MX_SR)
        return fail(MX_ERR_INVALID_ARG, "unknown rounding mode");
    if (cfg->hadamard != 0 && cfg->hadamard != 1) return fail(MX_ERR_INVALID_ARG, "hadamard must be 0 or 1");
    if (cfg->reserved != 0) return fail(MX_ERR_INVALID_ARG, "reserved field must be 0");
    if (cfg->scale_fmt == MX_SCALE_E8M0_TENSOR_F32 && !tensor_scale)
        return fail(MX_ERR_INVALID_ARG, "two-level scaling needs tensor_scale");
    if (cfg->scale_fmt == MX_SCALE_E8M0_TENSOR_F32 && (reinterpret_cast<uintptr_t>(tensor_scale) & 3u))
        return fail(MX_ERR_ALIGNMENT, "tensor_scale must be 4-byte aligned");
    return MX_OK;
}

mx_status check_source(const void* x, int32_t src, int64_t rows, int64_t cols, int64_t ld)
{
    if (!x) return fail(MX_ERR_INVALID_ARG, "x is NULL");
    if (src != MX_SRC_F32 && src != MX_SRC_BF16) return fail(MX_ERR_INVALID_ARG, "unknown source dtype");
    if (rows <= 0 || cols <= 0) return fail(MX_ERR_INVALID_ARG, "rows and cols must be > 0");
    if (ld < cols) return fail(MX_ERR_INVALID_ARG, "ld must be >= cols");
    const uintptr_t es = src == MX_SRC_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(x) % es != 0) return fail(MX_ERR_ALIGNMENT, "x must be aligned to its element size");
    return MX_OK;
}

mx::QuantJob make_job(const void* x, int32_t src, int64_t rows, int64_t cols, int64_t ld,
                      const mx_qconfig* cfg, float* tensor_scale)
{
    mx::QuantJob j{};
    j.x = x; j.src = src; j.rows = rows; j.cols = cols; j.ld = ld;
    j.fmt = cfg->fmt;
    j.sr = cfg->rounding == MX_SR;
    j.hadamard = cfg->hadamard != 0;
    j.two_level = cfg->scale_fmt == MX_SCALE_E8M0_TENSOR_F32 ? (cfg->tscale == MX_TSCALE_COMPUTE ? 1 : 2) : 0;
    j.seed = cfg->seed;
    j.offset = cfg->offset;
    j.tensor_scale = tensor_scale;
    return j;
}

}  // namespace

extern "C" {

const char* mx_status_string(mx_status s)
{
    switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARG: return "MX_ERR_INVALID_ARG";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_ALIGNMENT: return "MX_ERR_ALIGNMENT";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    }
    return "unknown mx_status";
}

const char* mx_last_error_message(void) { return g_msg; }

mx_status mx_quantize(const void* x, int32_t src_dtype, int64_t rows, int64_t cols, int64_t ld,
                      int32_t axis, const mx_qconfig* cfg, void* q, uint8_t* scales,
                      float* tensor_scale, void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_source(x, src_dtype, rows, cols, ld);
    if (s != MX_OK) return s;
    if ((s = check_cfg(cfg, tensor_scale)) != MX_OK) return s;
    if (!q || !scales) return fail(MX_ERR_INVALID_ARG, "q or scales is NULL");
    if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return fail(MX_ERR_INVALID_ARG, "unknown axis");
    if (axis == MX_AXIS_ROW && cols % 32 != 0) return fail(MX_ERR_INVALID_ARG, "row blocks need cols % 32 == 0");
    if (axis == MX_AXIS_COL && rows % 32 != 0) return fail(MX_ERR_INVALID_ARG, "column blocks need rows % 32 == 0");
    if (!aligned16(q)) return fail(MX_ERR_ALIGNMENT, "q must be 16-byte aligned");
    mx::QuantJob j = make_job(x, src_dtype, rows, cols, ld, cfg, tensor_scale);
    if (axis == MX_AXIS_ROW) { j.q_row = (uint8_t*)q; j.s_row = scales; }
    else { j.q_col = (uint8_t*)q; j.s_col = scales; }
    return hip_status(mx::launch_quantize(j, (hipStream_t)stream));
}

mx_status mx_quantize_dual_layout(const void* x, int32_t src_dtype, int64_t rows, int64_t cols,
                                  int64_t ld, const mx_qconfig* cfg, void* q_row,
                                  uint8_t* s_row, void* q_col, uint8_t* s_col,
                                  float* tensor_scale, void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_source(x, src_dtype, rows, cols, ld);
    if (s != MX_OK) return s;
    if ((s = check_cfg(cfg, tensor_scale)) != MX_OK) return s;
    if (!q_row || !s_row || !q_col || !s_col) return fail(MX_ERR_INVALID_ARG, "an output pointer is NULL");
    if (rows % 32 != 0 || cols % 32 != 0) return fail(MX_ERR_INVALID_ARG, "dual layout needs rows % 32 == 0 and cols % 32 == 0");
    if (!aligned16(q_row) || !aligned16(q_col)) return fail(MX_ERR_ALIGNMENT, "q_row and q_col must be 16-byte aligned");
    mx::QuantJob j = make_job(x, src_dtype, rows, cols, ld, cfg, tensor_scale);
    j.q_row = (uint8_t*)q_row; j.s_row = s_row;
    j.q_col = (uint8_t*)q_col; j.s_col = s_col;
    return hip_status(mx::launch_quantize(j, (hipStream_t)stream));
}

int64_t mx_predict_workspace_bytes(void) { return 4096; }

mx_status mx_predict_tensor_scale(const void* w, int64_t ld_w, const void* g, int64_t ld_g,
                                  int32_t src_dtype, int64_t rows, int64_t cols, float lr,
                                  int32_t fmt, void* work, int64_t work_bytes, float* scale_out,
                                  void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_source(w, src_dtype, rows, cols, ld_w);
    if (s != MX_OK) return s;
    if ((s = check_source(g, src_dtype, rows, cols, ld_g)) != MX_OK) return s;
    if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (!(lr >= 0.0f) || lr > 3.4028234663852886e38f) return fail(MX_ERR_INVALID_ARG, "lr must be finite and >= 0");
    if (!work || !scale_out) return fail(MX_ERR_INVALID_ARG, "work and scale_out must not be NULL");
    if (work_bytes < mx_predict_workspace_bytes()) return fail(MX_ERR_INVALID_ARG, "work is smaller than mx_predict_workspace_bytes()");
    if (((reinterpret_cast<uintptr_t>(work) | reinterpret_cast<uintptr_t>(scale_out)) & 3u) != 0)
        return fail(MX_ERR_ALIGNMENT, "work and scale_out must be 4-byte aligned");
    mx::PredictJob j{};
    j.w = w; j.g = g; j.src = src_dtype;
    j.rows = rows; j.cols = cols; j.ld_w = ld_w; j.ld_g = ld_g;
    j.lr = lr; j.fmt = fmt;
    j.work = (uint32_t*)work; j.scale_out = scale_out;
    return hip_status(mx::launch_predict(j, (hipStream_t)stream));
}

mx_status mx_predict_tensor_scale_noalloc(const void* w, int64_t ld_w, const void* g, int64_t ld_g,
                                          int32_t src_dtype, int64_t rows, int64_t cols, float lr,
                                          int32_t fmt, float* scale_out, void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_source(w, src_dtype, rows, cols, ld_w);
    if (s != MX_OK) return s;
    if ((s = check_source(g, src_dtype, rows, cols, ld_g)) != MX_OK) return s;
    if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (!(lr >= 0.0f) || lr > 3.4028234663852886e38f) return fail(MX_ERR_INVALID_ARG, "lr must be finite and >= 0");
    if (!scale_out) return fail(MX_ERR_INVALID_ARG, "scale_out must not be NULL");
    if (reinterpret_cast<uintptr_t>(scale_out) & 3u) return fail(MX_ERR_ALIGNMENT, "scale_out must be 4-byte aligned");
    mx::PredictJob j{};
    j.w = w; j.g = g; j.src = src_dtype;
    j.rows = rows; j.cols = cols; j.ld_w = ld_w; j.ld_g = ld_g;
    j.lr = lr; j.fmt = fmt;
    j.scale_out = scale_out;
    return hip_status(mx::launch_predict_noalloc(j, (hipStream_t)stream));
}

namespace {

mx_status check_optstate(int64_t n, int32_t group, int32_t fmt)
{
    if (fmt == MX_E2M1) return fail(MX_ERR_UNSUPPORTED, "optimizer states are quantized to FP8 (E4M3 or E5M2)");
    if (fmt != MX_E4M3 && fmt != MX_E5M2) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (group != 32 && group != 64 && group != 128 && group != 256)
        return fail(MX_ERR_INVALID_ARG, "group must be 32, 64, 128 or 256");
    if (n <= 0 || n % group != 0) return fail(MX_ERR_INVALID_ARG, "n must be a positive multiple of group");
    return MX_OK;
}

}  // namespace

mx_status mx_quantize_optstate(const float* x, int64_t n, int32_t group, int32_t fmt, uint8_t* q, float* amax,
                               float* kexp, void* stream)
{
    g_msg[0] = '\0';
    if (!x || !q || !amax || !kexp) return fail(MX_ERR_INVALID_ARG, "x, q, amax and kexp must not be NULL");
    mx_status s = check_optstate(n, group, fmt);
    if (s != MX_OK) return s;
    if (!aligned16(x)) return fail(MX_ERR_ALIGNMENT, "x must be 16-byte aligned");
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(amax) | reinterpret_cast<uintptr_t>(kexp)) & 3u) != 0)
        return fail(MX_ERR_ALIGNMENT, "q, amax and kexp must be 4-byte aligned");
    mx::OptStateJob j{};
    j.x = x; j.n = n; j.group = group; j.fmt = fmt; j.dequant = false;
    j.q = q; j.amax = amax; j.k = kexp;
    return hip_status(mx::launch_optstate(j, (hipStream_t)stream));
}

mx_status mx_dequantize_optstate(const uint8_t* q, const float* amax, const float* kexp, int64_t n, int32_t group,
                                 int32_t fmt, float* out, void* stream)
{
    g_msg[0] = '\0';
    if (!q || !amax || !kexp || !out) return fail(MX_ERR_INVALID_ARG, "q, amax, kexp and out must not be NULL");
    mx_status s = check_optstate(n, group, fmt);
    if (s != MX_OK) return s;
    if (!aligned16(out)) return fail(MX_ERR_ALIGNMENT, "out must be 16-byte aligned");
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(amax) | reinterpret_cast<uintptr_t>(kexp)) & 3u) != 0)
        return fail(MX_ERR_ALIGNMENT, "q, amax and kexp must be 4-byte aligned");
    mx::OptStateJob j{};
    j.n = n; j.group = group; j.fmt = fmt; j.dequant = true;
    j.q = (uint8_t*)q; j.amax = (float*)amax; j.k = (float*)kexp; j.out = out;
    return hip_status(mx::launch_optstate(j, (hipStream_t)stream));
}

namespace {

// stored rows and their length of one nvfp copy
void nv_dims(int64_t rows, int64_t cols, int32_t axis, int64_t* SR, int64_t* L)
{
    *SR = axis == MX_AXIS_ROW ? rows : cols;
    *L = axis == MX_AXIS_ROW ? cols : rows;
}

mx_status check_nv_copy(int64_t rows, int64_t cols, int32_t axis, int32_t local)
{
    if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return fail(MX_ERR_INVALID_ARG, "unknown axis");
    if (local != 0 && local != 1) return fail(MX_ERR_INVALID_ARG, "local must be 0 or 1");
    if (rows <= 0 || cols <= 0) return fail(MX_ERR_INVALID_ARG, "rows and cols must be > 0");
    int64_t SR, L;
    nv_dims(rows, cols, axis, &SR, &L);
    if (L % 16 != 0) return fail(MX_ERR_INVALID_ARG, "the blocked dimension must be a multiple of 16");
    return MX_OK;
}

}  // namespace

mx_status mx_quantize_nvfp(const void* x, int32_t src_dtype, int64_t rows, int64_t cols, int64_t ld,
                           int32_t axis, int32_t local, uint8_t* q, uint8_t* scales, float* tscale,
                           void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_source(x, src_dtype, rows, cols, ld);
    if (s != MX_OK) return s;
    if ((s = check_nv_copy(rows, cols, axis, local)) != MX_OK) return s;
    if (!q || !scales || !tscale) return fail(MX_ERR_INVALID_ARG, "q, scales and tscale must not be NULL");
    if (!aligned16(q)) return fail(MX_ERR_ALIGNMENT, "q must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(tscale) & 3u) return fail(MX_ERR_ALIGNMENT, "tscale must be 4-byte aligned");
    mx::NvQuantJob j{};
    j.x = x; j.src = src_dtype; j.rows = rows; j.cols = cols; j.ld = ld; j.axis = axis; j.local = local;
    j.q = q; j.s16 = scales; j.ts = tscale;
    return hip_status(mx::launch_nv_quantize(j, (hipStream_t)stream));
}

mx_status mx_dequantize_nvfp(const uint8_t* q, const uint8_t* scales, const float* tscale, int64_t rows,
                             int64_t cols, int32_t axis, int32_t local, void* out, int32_t out_dtype,
                             void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_nv_copy(rows, cols, axis, local);
    if (s != MX_OK) return s;
    if (!q || !scales || !tscale || !out) return fail(MX_ERR_INVALID_ARG, "q, scales, tscale and out must not be NULL");
    if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return fail(MX_ERR_INVALID_ARG, "unknown output dtype");
    if (!aligned16(q)) return fail(MX_ERR_ALIGNMENT, "q must be 16-byte aligned");
    const uintptr_t es = out_dtype == MX_OUT_F32 ? 4 : 2;
    if (reinterpret_cast<uintptr_t>(out) % es != 0) return fail(MX_ERR_ALIGNMENT, "out must be aligned to its element size");
    if (reinterpret_cast<uintptr_t>(tscale) & 3u) return fail(MX_ERR_ALIGNMENT, "tscale must be 4-byte aligned");
    mx::NvQuantJob j{};
    j.rows = rows; j.cols = cols; j.axis = axis; j.local = local;
    j.q = (uint8_t*)q; j.s16 = (uint8_t*)scales; j.ts = (float*)tscale;
    return hip_status(mx::launch_nv_dequantize(j, out, out_dtype, (hipStream_t)stream));
}

mx_status mx_gemm_nvfp(const uint8_t* qa, const uint8_t* sa, const float* ta, int32_t local_a,
                       const uint8_t* qb, const uint8_t* sb, const float* tb, int32_t local_b,
                       int64_t M, int64_t N, int64_t K, float alpha, void* c, int32_t out_dtype,
                       int64_t ldc, void* stream)
{
    g_msg[0] = '\0';
    if (!qa || !sa || !ta || !qb || !sb || !tb || !c) return fail(MX_ERR_INVALID_ARG, "an operand pointer is NULL");
    if ((local_a != 0 && local_a != 1) || (local_b != 0 && local_b != 1))
        return fail(MX_ERR_INVALID_ARG, "local_a and local_b must be 0 or 1");
    if (M <= 0 || N <= 0 || K <= 0) return fail(MX_ERR_INVALID_ARG, "M, N, K must be > 0");
    if (K % 64 != 0) return fail(MX_ERR_INVALID_ARG, "K must be a multiple of 64");
    if (K > (int64_t)1 << 24) return fail(MX_ERR_INVALID_ARG, "K must be <= 2^24");
    if (M > ((int64_t)1 << 31) - 256 || N > ((int64_t)1 << 31) - 256) return fail(MX_ERR_INVALID_ARG, "M and N must be < 2^31 - 256");
    if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t)1 << 31)
        return fail(MX_ERR_INVALID_ARG, "M x N must be fewer than 2^31 output tiles of 256 x 256");
    if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return fail(MX_ERR_INVALID_ARG, "unknown output dtype");
    if (ldc < N) return fail(MX_ERR_INVALID_ARG, "ldc must be >= N");
    if (!aligned16(qa) || !aligned16(qb)) return fail(MX_ERR_ALIGNMENT, "qa and qb must be 16-byte aligned");
    if (((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sb) | reinterpret_cast<uintptr_t>(ta) |
          reinterpret_cast<uintptr_t>(tb)) & 3u) != 0)
        return fail(MX_ERR_ALIGNMENT, "sa, sb, ta and tb must be 4-byte aligned");
    const uintptr_t es = out_dtype == MX_OUT_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(c) % es) != 0) return fail(MX_ERR_ALIGNMENT, "c must be aligned to its element size");
    mx::NvGemmJob j{};
    j.qa = qa; j.sa = sa; j.ta = ta; j.la = local_a;
    j.qb = qb; j.sb = sb; j.tb = tb; j.lb = local_b;
    j.M = M; j.N = N; j.K = K; j.alpha = alpha;
    j.c = c; j.out_dtype = out_dtype; j.ldc = ldc;
    return hip_status(mx::launch_nv_gemm(j, (hipStream_t)stream));
}

namespace {

mx_status check_gemm_operands(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                              const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                              int64_t M, int64_t N, int64_t K, int32_t hadamard_k)
{
    if (!qa || !sa || !qb || !sb) return fail(MX_ERR_INVALID_ARG, "an operand pointer is NULL");
    if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (M <= 0 || N <= 0 || K <= 0) return fail(MX_ERR_INVALID_ARG, "M, N, K must be > 0");
    if (K % 32 != 0) return fail(MX_ERR_INVALID_ARG, "K must be a multiple of 32");
    // the kernels address a 256-row operand tile with 32-bit offsets from its
    // first row, and number their workgroups with 32-bit integers
    if (K > (int64_t)1 << 23) return fail(MX_ERR_INVALID_ARG, "K must be <= 2^23");
    if (M > ((int64_t)1 << 31) - 256 || N > ((int64_t)1 << 31) - 256) return fail(MX_ERR_INVALID_ARG, "M and N must be < 2^31 - 256");
    if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t)1 << 31)
        return fail(MX_ERR_INVALID_ARG, "M x N must be fewer than 2^31 output tiles of 256 x 256");
    if (hadamard_k != 0 && hadamard_k != 1) return fail(MX_ERR_INVALID_ARG, "hadamard_k must be 0 or 1");
    if (elem_bits(fa) != elem_bits(fb)) return fail(MX_ERR_UNSUPPORTED, "mixed FP8 x FP4 operands are not built");
    if (!aligned16(qa) || !aligned16(qb)) return fail(MX_ERR_ALIGNMENT, "qa and qb must be 16-byte aligned");
    if (((reinterpret_cast<uintptr_t>(ta) | reinterpret_cast<uintptr_t>(tb)) & 3u) != 0)
        return fail(MX_ERR_ALIGNMENT, "ta and tb must be 4-byte aligned");
    return MX_OK;
}

mx::GemmJob gemm_job(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                     const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                     int64_t M, int64_t N, int64_t K, float alpha, int32_t hadamard_k)
{
    mx::GemmJob j{};
    j.qa = (const uint8_t*)qa; j.sa = sa; j.ta = ta; j.fa = fa;
    j.qb = (const uint8_t*)qb; j.sb = sb; j.tb = tb; j.fb = fb;
    j.M = M; j.N = N; j.K = K;
    j.alpha = alpha; j.hadamard_k = hadamard_k != 0;
    return j;
}

}  // namespace

mx_status mx_gemm(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                  const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                  int64_t M, int64_t N, int64_t K, float alpha, int32_t hadamard_k,
                  void* c, int32_t out_dtype, int64_t ldc, void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_gemm_operands(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, hadamard_k);
    if (s != MX_OK) return s;
    if (!c) return fail(MX_ERR_INVALID_ARG, "an operand pointer is NULL");
    if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return fail(MX_ERR_INVALID_ARG, "unknown output dtype");
    if (ldc < N) return fail(MX_ERR_INVALID_ARG, "ldc must be >= N");
    const uintptr_t es = out_dtype == MX_OUT_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(c) % es) != 0) return fail(MX_ERR_ALIGNMENT, "c must be aligned to its element size");
    mx::GemmJob j = gemm_job(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha, hadamard_k);
    j.c = c; j.out_dtype = out_dtype; j.ldc = ldc;
    return hip_status(mx::launch_gemm(j, (hipStream_t)stream));
}

mx_status mx_gemm_quantized(const void* qa, const uint8_t* sa, const float* ta, int32_t fa,
                            const void* qb, const uint8_t* sb, const float* tb, int32_t fb,
                            int64_t M, int64_t N, int64_t K, float alpha, int32_t hadamard_k,
                            int32_t out_fmt, void* qc, uint8_t* sc, void* stream)
{
    g_msg[0] = '\0';
    mx_status s = check_gemm_operands(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, hadamard_k);
    if (s != MX_OK) return s;
    if (!qc || !sc) return fail(MX_ERR_INVALID_ARG, "qc and sc must not be NULL");
    if (!valid_fmt(out_fmt)) return fail(MX_ERR_INVALID_ARG, "unknown output element format");
    if (out_fmt == MX_E2M1) return fail(MX_ERR_UNSUPPORTED, "the quantized GEMM output is FP8 (E4M3 or E5M2)");
    if (N % 32 != 0) return fail(MX_ERR_INVALID_ARG, "N must be a multiple of 32 (1x32 output blocks)");
    if (!aligned16(qc)) return fail(MX_ERR_ALIGNMENT, "qc must be 16-byte aligned");
    mx::GemmJob j = gemm_job(qa, sa, ta, fa, qb, sb, tb, fb, M, N, K, alpha, hadamard_k);
    j.c = qc; j.cs = sc; j.ldc = N;
    j.out_dtype = out_fmt == MX_E4M3 ? 2 : 3;
    if (!mx::gemm_w4_eligible(j))
        return fail(MX_ERR_UNSUPPORTED, "the quantized output needs rows of K holding a multiple of 128 bytes of "
                                        "codes (FP8: K % 128 == 0, FP4: K % 256 == 0) and 4-byte aligned sa, sb");
    return hip_status(mx::launch_gemm(j, (hipStream_t)stream));
}

mx_status mx_dequantize(const void* q, const uint8_t* scales, const float* tensor_scale,
                        int32_t fmt, int64_t rows, int64_t cols, int32_t axis, int32_t hadamard,
                        void* out, int32_t out_dtype, void* stream)
{
    g_msg[0] = '\0';
    if (!q || !scales || !out) return fail(MX_ERR_INVALID_ARG, "q, scales or out is NULL");
    if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "unknown element format");
    if (axis != MX_AXIS_ROW && axis != MX_AXIS_COL) return fail(MX_ERR_INVALID_ARG, "unknown axis");
    if (hadamard != 0 && hadamard != 1) return fail(MX_ERR_INVALID_ARG, "hadamard must be 0 or 1");
    if (out_dtype != MX_OUT_F32 && out_dtype != MX_OUT_BF16) return fail(MX_ERR_INVALID_ARG, "unknown output dtype");
    if (rows <= 0 || cols <= 0) return fail(MX_ERR_INVALID_ARG, "rows and cols must be > 0");
    if (axis == MX_AXIS_ROW && cols % 32 != 0) return fail(MX_ERR_INVALID_ARG, "row blocks need cols % 32 == 0");
    if (axis == MX_AXIS_COL && rows % 32 != 0) return fail(MX_ERR_INVALID_ARG, "column blocks need rows % 32 == 0");
    if (!aligned16(q) || !aligned16(out)) return fail(MX_ERR_ALIGNMENT, "q and out must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(tensor_scale) & 3u) return fail(MX_ERR_ALIGNMENT, "tensor_scale must be 4-byte aligned");
    mx::DequantJob j{};
    j.q = (const uint8_t*)q; j.scales = scales; j.tensor_scale = tensor_scale;
    j.fmt = fmt; j.rows = rows; j.cols = cols; j.axis = axis; j.hadamard = hadamard != 0;
    j.out = out; j.out_dtype = out_dtype;
    return hip_status(mx::launch_dequantize(j, (hipStream_t)stream));
}

}  // extern "C"
