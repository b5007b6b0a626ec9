// MXFP8 quantization of a BF16 matrix along its rows for gfx950 (Sol-H3
// report, §3.3 "Compute Quantization", "MXFP8 GEMM computation": E4M3 values
// with one E8M0 scale per 32 values along the reduction dimension).
//
// Per group of 32 consecutive values of a row: amax = max |x|, the shared
// exponent e = floor(log2 amax) - 8 (read from amax's FP32 exponent field,
// clamped below at -127; a zero group takes -127), and each element is
// x * 2^-e (exact in FP32) clamped to +-448 and rounded to the nearest E4M3
// value, ties to even, by the hardware conversion. The scale code is e + 127.
// Scales are stored K-slab-major, scales[k / 128][row][4], the layout the
// MXFP8 GEMM loads a stage at a time.
//
// 16 lanes cover one 128-wide slab of one row with coalesced 16-byte loads
// (8 values per lane); a group is 4 lanes, reduced with two lane swaps; the
// first lane of the 16 gathers the slab's 4 scale codes into one dword.
// Padding rows [rows_valid, rows_buf) get zero codes and zero scale codes.
#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t *x, int64_t ld_x, int64_t rows_buf,
                                                          int64_t rows_valid, int32_t slabs, uint8_t *q,
                                                          int64_t ld_q, uint8_t *scales) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int l16 = (int)(gid & 15);
    const int64_t item = gid >> 4;
    if (item >= rows_buf * slabs) return;  // whole 16-lane teams only (blockDim is a multiple of 16)
    const int64_t row = item / slabs;
    const int slab = (int)(item - row * slabs);
    const int64_t col = (int64_t)slab * 128 + 8 * l16;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < rows_valid) unpack8(*reinterpret_cast<const uint4 *>(x + row * ld_x + col), f);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int ex = mx_shared_exponent(amax);
    const float inv = mx_inv_scale(ex);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = f[e] * inv;
    *reinterpret_cast<uint2 *>(q + row * ld_q + col) = e4m3x8(y);
    // scale codes of the slab's 4 groups (lanes 0, 4, 8, 12 of the team)
    const uint32_t code = (uint32_t)(ex + 127);
    const uint32_t c1 = __shfl_down(code, 4), c2 = __shfl_down(code, 8), c3 = __shfl_down(code, 12);
    if (l16 == 0)
        *reinterpret_cast<uint32_t *>(scales + ((int64_t)slab * rows_buf + row) * 4) =
            code | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Zero codes and scale codes of rows [r0, r1) of an MXFP8 matrix with `slabs`
// 128-wide scale slabs and rows_buf scale rows.
__global__ __launch_bounds__(256) void mx_zero_rows_kernel(uint8_t *q, int64_t ld_q, int32_t slabs, uint8_t *scales,
                                                           int64_t rows_buf, int64_t r0, int64_t r1) {
    const int64_t r = r0 + blockIdx.x;
    if (r >= r1) return;
    for (int c = threadIdx.x; c < slabs * 8; c += blockDim.x)
        *reinterpret_cast<uint4 *>(q + r * ld_q + 16 * c) = make_uint4(0, 0, 0, 0);
    for (int k = threadIdx.x; k < slabs; k += blockDim.x)
        *reinterpret_cast<uint32_t *>(scales + ((int64_t)k * rows_buf + r) * 4) = 0;
}

}  // namespace

void launch_mx_zero_rows(uint8_t *q, int64_t ld_q, int64_t K, uint8_t *scales, int64_t rows_buf, int64_t r0,
                         int64_t r1, hipStream_t stream) {
    if (r1 <= r0) return;
    mx_zero_rows_kernel<<<dim3((unsigned)(r1 - r0)), 256, 0, stream>>>(q, ld_q, (int32_t)(K / 128), scales, rows_buf,
                                                                      r0, r1);
}

void launch_mx_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K, uint8_t *q,
                        int64_t ld_q, uint8_t *scales, hipStream_t stream) {
    const int32_t slabs = (int32_t)(K / 128);
    const int64_t threads = rows_buf * slabs * 16;
    if (threads == 0) return;
    mx_quantize_kernel<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, stream>>>(x, ld_x, rows_buf, rows_valid,
                                                                                    slabs, q, ld_q, scales);
}

}  // namespace h3

using namespace h3;

extern "C" int h3_mxfp8_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K,
                                 uint8_t *q, int64_t ld_q, uint8_t *scales, void *stream) {
    int s = h3_check_mxfp8_quantize(x, ld_x, rows_buf, rows_valid, K, q, ld_q, scales);
    if (s != H3_OK || rows_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_mx_quantize(x, ld_x, rows_buf, rows_valid, K, q, ld_q, scales, (hipStream_t)stream);
    return launch_status();
}
