// A measured ceiling for the matrix-core roofline: the rate at which one
// gfx950 sustains v_mfma_f32_32x32x16_bf16 (or the MXFP8 scaled MFMA) in the register pattern of this
// library's GEMM tile (4 A and 4 B operands per wave, 16 independent 32x32
// accumulators, c[i][j] += a[i] b[j]) on BF16 operands whose bits vary like
// real data (uniform in [-1, 1)), with no memory traffic at all. Under load
// the chip's clock is set by power, and power depends on how many operand
// bits toggle: on constant operands the same loop runs at the full clock,
// on varying ones it does not, so this figure, not the published peak,
// bounds what a kernel on such data can reach.
#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int kCeilThreads = 256;

// An integer mix (xorshift-multiply rounds) giving operand bits per lane.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// The same pattern on the MXFP8 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
// E4M3 operands, unit E8M0 scales), whose issue rate is twice BF16's per
// flop: random E4M3 codes with the exponent kept below all-ones (no NaN).
__global__ __launch_bounds__(kCeilThreads, 1) void mfma_ceiling_fp8_kernel(float *sink, int32_t iters) {
    i32x8_t a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h1 = mix32(threadIdx.x * 131u + blockIdx.x * 7919u + (uint32_t)(s * 31 + e));
            const uint32_t h2 = mix32(h1 + 12345u);
            a[s][e] = (int)(h1 & 0xF7F7F7F7u);
            b[s][e] = (int)(h2 & 0xF7F7F7F7u);
        }
    const int unit = 0x7F7F7F7F;  // E8M0 127 = 2^0 in every byte
    f32x16_t c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) c[i][j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                c[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], c[i][j], 0, 0, 0, unit, 0, unit);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += c[i][j][e];
    sink[(int64_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kCeilThreads, 1) void mfma_ceiling_kernel(float *sink, int32_t iters) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h1 = mix32(threadIdx.x * 131u + blockIdx.x * 7919u + (uint32_t)(s * 31 + e));
            const uint32_t h2 = mix32(h1 + 12345u);
            a[s][e] = (__bf16)((float)(h1 & 0xffffu) * (1.0f / 32768.0f) - 1.0f);
            b[s][e] = (__bf16)((float)(h2 & 0xffffu) * (1.0f / 32768.0f) - 1.0f);
        }
    f32x16_t c[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) c[i][j][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], c[i][j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += c[i][j][e];
    sink[(int64_t)blockIdx.x * kCeilThreads + threadIdx.x] = s;  // keeps the products live
}

}  // namespace
}  // namespace h3

using namespace h3;

extern "C" int h3_mfma_ceiling(int32_t dtype, int32_t iters, float *sink, int64_t sink_floats, double *flops,
                               void *stream) {
    int s = h3_check_mfma_ceiling(dtype, iters, sink, sink_floats, flops);
    if (s != H3_OK) return s;
    if ((s = device_check()) != H3_OK) return s;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) return H3_ERR_HIP;
    if (sink_floats < (int64_t)cus * kCeilThreads) return H3_ERR_SHAPE;
    // one workgroup of 4 waves per CU; each wave issues 16 MFMAs per iteration, of 2*32*32*16 flops (BF16)
    // or 2*32*32*64 (FP8)
    *flops = (double)cus * 4.0 * (double)iters * 16.0 * (dtype == H3_CEIL_FP8 ? 131072.0 : 32768.0);
    if (dtype == H3_CEIL_FP8)
        mfma_ceiling_fp8_kernel<<<dim3((unsigned)cus), kCeilThreads, 0, (hipStream_t)stream>>>(sink, iters);
    else
        mfma_ceiling_kernel<<<dim3((unsigned)cus), kCeilThreads, 0, (hipStream_t)stream>>>(sink, iters);
    return launch_status();
}
