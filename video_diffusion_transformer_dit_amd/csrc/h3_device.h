// Device-side helpers shared by the gfx950 kernels of libh3block.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace h3 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (4 SGPRs) over `bytes` bytes from `base` (clamped to
// 4 GiB), wave-uniform by construction: loads past the end return zero.
__device__ __forceinline__ i32x4_t raw_rsrc(const void *base, int64_t bytes) {
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r.x = (int)__builtin_amdgcn_readfirstlane((uint32_t)addr);
    r.y = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32)) & 0xFFFFu);  // stride 0
    r.z = (int)__builtin_amdgcn_readfirstlane(bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    r.w = 0x00020000;
    return r;
}

// LDS byte address of a __shared__ object, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}

// Direct global -> LDS load of one 1 KB slab: lane i's 16 bytes (descriptor
// rsrc, byte offset voff + soff) land at LDS address lds + 16 i. Issued as one
// asm statement (M0 set, the M0 -> LDS-DMA wait state, the load) so the
// compiler neither reuses M0 in between nor inserts its conservative
// "may alias any LDS read" waits: callers order these loads themselves with
// s_waitcnt vmcnt and a barrier before reading the slab.
__device__ __forceinline__ void dma_slab(i32x4_t rsrc, uint32_t lds, int voff, int soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory", "m0");
}

// Direct global -> LDS load of 4 bytes per lane: lane i's dword (descriptor
// rsrc, byte offset voff + soff) lands at LDS address lds + 4 i. Same
// ordering contract as dma_slab.
__device__ __forceinline__ void dma_dword(i32x4_t rsrc, uint32_t lds, int voff, int soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, %3 offen lds"
        :
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory", "m0");
}

// GEMM tile order. The grouped order walks group_m tile rows at a time,
// column by column; gemm_grouped_coords maps a position in it to (tile_m,
// tile_n).
__device__ __forceinline__ void gemm_grouped_coords(int lin, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
    const int per_group = group_m * tiles_n;
    const int group = lin / per_group;
    const int first_m = group * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in_group = lin - group * per_group;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
}
// Workgroup id -> tile among the first T tiles of the grouped order, such that
// each XCD (workgroups are dealt round-robin over 8 XCDs) walks a contiguous
// range of that order.
__device__ __forceinline__ void gemm_tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int T, int &tm,
                                                 int &tn) {
    const int q = T / 8, rr = T % 8;
    const int xcd = bid % 8, local = bid / 8;
    const int lin = xcd < rr ? xcd * (q + 1) + local : rr * (q + 1) + (xcd - rr) * q + local;
    gemm_grouped_coords(lin, tiles_m, tiles_n, group_m, tm, tn);
}
__device__ __forceinline__ void gemm_tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
    gemm_tile_coords(bid, tiles_m, tiles_n, group_m, tiles_m * tiles_n, tm, tn);
}

// ---- MXFP8 (E4M3 elements, one E8M0 scale per 32 values) ----
// Shared exponent of a group from its largest magnitude: floor(log2 amax) - 8,
// read from amax's FP32 exponent field, clamped below at -127 (zero and FP32
// subnormal groups get -127). The scale code is this + 127.
__device__ __forceinline__ int mx_shared_exponent(float amax) {
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    return max(eb - 127 - 8, -127);
}
// 2^-e as a float, exact for the exponents mx_shared_exponent returns.
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
// 8 floats, already divided by the group scale, -> 8 E4M3 codes: saturate to
// +-448, then the hardware conversion (round to nearest, ties to even).
__device__ __forceinline__ uint2 e4m3x8(const float y[8]) {
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = fminf(fmaxf(y[e], -448.0f), 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.0f), 448.0f), fminf(fmaxf(b, -448.0f), 448.0f), 0,
                                            false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -448.0f), 448.0f), fminf(fmaxf(d, -448.0f), 448.0f), v, true);
    return (uint32_t)v;
}

// 16-byte global load / store with the non-temporal hint, for data a kernel
// streams once (measured on the modulate-norm pass: 4.9 -> 5.2 TB/s).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const void *p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(void *p, const uint4 &v) {
    const u32x4_nt w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt *>(p));
}

// BF16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
// SiLU, x / (1 + e^-x), with the hardware reciprocal (v_rcp_f32, within 1 ulp)
// in place of an IEEE divide (about ten instructions): every caller rounds the
// result to BF16 or E4M3 right after, far coarser than that ulp. A large
// negative x (e^-x overflowing to inf) gives a reciprocal of 0 and a product
// of -0, as the divide would; NaN propagates.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// 8 BF16 values in one 128-bit word <-> 8 floats.
__device__ __forceinline__ void unpack8(const uint4 &u, float f[8]) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
__device__ __forceinline__ uint4 pack8(const float f[8]) {
    uint4 u;
    u.x = pack_bf16x2(f[0], f[1]);
    u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]);
    u.w = pack_bf16x2(f[6], f[7]);
    return u;
}

// Sum over the 64 lanes of a wavefront (every lane receives the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Sum over aligned groups of 16 lanes.
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

}  // namespace h3
