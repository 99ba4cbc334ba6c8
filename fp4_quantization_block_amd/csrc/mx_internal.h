// mx_internal.h -- host-side launchers shared by the ABI layer and the
// kernel translation units.  Every launcher assumes its arguments were
// validated by the ABI layer and returns the hipError_t of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

struct QuantJob {
    const void* x;          // source tile, row stride ld elements
    int src;                // SRC_F32 / SRC_BF16
    int64_t rows, cols, ld;
    int fmt;                // E4M3 / E5M2 / E2M1
    bool sr, hadamard;
    int two_level;          // 0 none, 1 s_t from the amax word, 2 s_t provided
    uint64_t seed;
    uint32_t offset;
    uint8_t* q_row;  uint8_t* s_row;    // row copy (nullptr: not written)
    uint8_t* q_col;  uint8_t* s_col;    // column copy (nullptr: not written)
    float* tensor_scale;    // two-level: amax scratch / s_t
};

hipError_t launch_quantize(const QuantJob& j, hipStream_t stream);

// predicted per-tensor scale from W and g (weight auto-scaling)
struct PredictJob {
    const void* w; const void* g;
    int src;                // SRC_F32 / SRC_BF16
    int64_t rows, cols, ld_w, ld_g;
    float lr;
    int fmt;
    uint32_t* work;         // >= 1024 words of caller workspace
    float* scale_out;
};

hipError_t launch_predict(const PredictJob& j, hipStream_t stream);
// the same with the library's own per-device scratch in place of j.work
hipError_t launch_predict_noalloc(PredictJob j, hipStream_t stream);

// FP8 optimizer states with dynamic range expansion: quantize (x -> q,
// amax, k) or dequantize (q, amax, k -> out); n elements, group size G
struct OptStateJob {
    const float* x; int64_t n; int group; int fmt; bool dequant;
    uint8_t* q; float* amax; float* k; float* out;
};

hipError_t launch_optstate(const OptStateJob& j, hipStream_t stream);

// nvfp routes: NVFP4 copies (E2M1, E4M3 scale per 16, FP32 second-level
// scale over the tensor or per 32 stored rows)
struct NvQuantJob {
    const void* x; int src; int64_t rows, cols, ld; int axis; int local;
    uint8_t* q; uint8_t* s16; float* ts;
};

hipError_t launch_nv_quantize(const NvQuantJob& j, hipStream_t stream);
hipError_t launch_nv_dequantize(const NvQuantJob& j, const void* out, int out_dtype, hipStream_t stream);

struct NvGemmJob {
    const uint8_t* qa; const uint8_t* sa; const float* ta; int la;
    const uint8_t* qb; const uint8_t* sb; const float* tb; int lb;
    int64_t M, N, K; float alpha;
    void* c; int out_dtype; int64_t ldc;
};

hipError_t launch_nv_gemm(const NvGemmJob& j, hipStream_t stream);

struct DequantJob {
    const uint8_t* q; const uint8_t* scales; const float* tensor_scale;
    int fmt; int64_t rows, cols; int axis; bool hadamard;
    void* out; int out_dtype;
};

hipError_t launch_dequantize(const DequantJob& j, hipStream_t stream);

struct GemmJob {
    const uint8_t* qa; const uint8_t* sa; const float* ta; int fa;
    const uint8_t* qb; const uint8_t* sb; const float* tb; int fb;
    int64_t M, N, K;
    float alpha; bool hadamard_k;
    void* c; int out_dtype; int64_t ldc;   // out_dtype 0 f32, 1 bf16, 2 MX E4M3 codes, 3 MX E5M2 codes
    uint8_t* cs;                            // MX output: [M][N/32] scale bytes
};

hipError_t launch_gemm(const GemmJob& j, hipStream_t stream);

// whether launch_gemm takes the one-wave-per-SIMD kernel (the only one with
// the MX-quantized output): rows of K holding a multiple of 128 bytes of
// codes, 4-byte aligned scale arrays
bool gemm_w4_eligible(const GemmJob& j);

}  // namespace mx
