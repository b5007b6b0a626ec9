// Epilogue shared by the block's GEMM kernels (BF16 and MXFP8 operands):
// the FP32 accumulators of one 256 x 256 output tile, held by 4 wavefronts
// of 128 x 128 as 4 x 4 MFMA sub-tiles of 32 x 32 (weight tile = MFMA A
// operand, activation tile = B operand), become BF16 outputs.
//   H3_EPI_STORE     c = acc + bias
//   H3_EPI_RESIDUAL  c = resid + gate[i] * (acc + bias)   (Sol-H3 report, §3.5
//                    "Kernel Fusion", group (1): residual with indexed gating)
//   H3_EPI_SWIGLU    c = silu(acc_gate + b) * (acc_up + b)   (group (3)); the
//                    weight tile interleaves 16-row gate and up blocks
#pragma once

#include "h3_device.h"
#include "h3block.h"

namespace h3 {

// Internal epilogue: SwiGLU with its output written as MXFP8 (E4M3 codes at
// p.cq / p.ld_cq, scale codes at p.cs with p.cs_rows scale rows), the fused
// quantizing SwiGLU producer of Sol-H3 report, §3.3 "MXFP8 GEMM computation".
constexpr int kEpiSwigluMx = 3;

// In each 32 x 32 sub-tile the lane holds row m = lane & 31 and, for register
// group q (0..3), the 4 columns 8 q + 4 (lane >> 5) + (0..3). Args provides
// M, N, ffn, c/ldc, bias, resid/ld_r, gate/ld_gate, mod_idx and n_groups.
template <int EPI, typename Args>
__device__ __forceinline__ void gemm_epilogue(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn, int wm, int wn,
                                              int r32, int g2) {
    constexpr int BM = 256, BN = 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = (int64_t)tm * BM + wm * 128 + j * 32 + r32;
        if (m >= p.M) continue;
        uint16_t *crow = EPI == kEpiSwigluMx ? nullptr : p.c + m * p.ldc;
        if constexpr (EPI == kEpiSwigluMx) {
            // A 32-wide output group is W sub-tiles i = 2 ip, 2 ip + 1: 16
            // values in this lane (4 columns x q x 2 sub-tiles) and 16 in lane
            // ^ 32 (the other 4-column halves).
#pragma unroll
            for (int ip = 0; ip < 2; ++ip) {
                const int64_t col0 = (int64_t)tn * (BN / 2) + (wn * 4 + 2 * ip) * 16;
                if (col0 >= p.ffn) continue;
                float o[2][2][4];
                float amax = 0.f;
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = 2 * ip + ii;
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int64_t col = col0 + 16 * ii + 8 * q + 4 * g2;
                        float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
                        if (p.bias) {
                            const uint2 bg = *reinterpret_cast<const uint2 *>(p.bias + col);
                            const uint2 bu = *reinterpret_cast<const uint2 *>(p.bias + p.ffn + col);
                            gb[0] = bf16_lo(bg.x); gb[1] = bf16_hi(bg.x); gb[2] = bf16_lo(bg.y); gb[3] = bf16_hi(bg.y);
                            ub[0] = bf16_lo(bu.x); ub[1] = bf16_hi(bu.x); ub[2] = bf16_lo(bu.y); ub[3] = bf16_hi(bu.y);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float zg = acc[i][j][4 * q + e] + gb[e];
                            o[ii][q][e] = zg / (1.0f + __expf(-zg)) * (acc[i][j][4 * (q + 2) + e] + ub[e]);
                            amax = fmaxf(amax, fabsf(o[ii][q][e]));
                        }
                    }
                }
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                const int ex = mx_shared_exponent(amax);
                const float is = mx_inv_scale(ex);
                uint8_t *qrow = p.cq + m * p.ld_cq;
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        *reinterpret_cast<uint32_t *>(qrow + col0 + 16 * ii + 8 * q + 4 * g2) =
                            e4m3x4(o[ii][q][0] * is, o[ii][q][1] * is, o[ii][q][2] * is, o[ii][q][3] * is);
                if (g2 == 0) p.cs[((col0 >> 7) * p.cs_rows + m) * 4 + ((col0 >> 5) & 3)] = (uint8_t)(ex + 127);
            }
        } else if (EPI == H3_EPI_SWIGLU) {
            // W sub-tile i holds the gate block (rows 0-15, q = 0, 1) and the up
            // block (rows 16-31, q = 2, 3) of output columns (wn*4 + i)*16 + 0..15.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int64_t col = (int64_t)tn * (BN / 2) + (wn * 4 + i) * 16 + 8 * q + 4 * g2;
                    if (col >= p.ffn) continue;
                    float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
                    if (p.bias) {
                        const uint2 bg = *reinterpret_cast<const uint2 *>(p.bias + col);
                        const uint2 bu = *reinterpret_cast<const uint2 *>(p.bias + p.ffn + col);
                        gb[0] = bf16_lo(bg.x); gb[1] = bf16_hi(bg.x); gb[2] = bf16_lo(bg.y); gb[3] = bf16_hi(bg.y);
                        ub[0] = bf16_lo(bu.x); ub[1] = bf16_hi(bu.x); ub[2] = bf16_lo(bu.y); ub[3] = bf16_hi(bu.y);
                    }
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float zg = acc[i][j][4 * q + e] + gb[e];
                        o[e] = zg / (1.0f + __expf(-zg)) * (acc[i][j][4 * (q + 2) + e] + ub[e]);
                    }
                    *reinterpret_cast<uint2 *>(crow + col) =
                        make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                }
            }
        } else {
            const float *grow = nullptr;
            const uint16_t *rrow = nullptr;
            if (EPI == H3_EPI_RESIDUAL) {
                int g = 0;
                if (p.mod_idx) g = min(max(p.mod_idx[m], 0), p.n_groups - 1);
                grow = p.gate + (int64_t)g * p.ld_gate;
                rrow = p.resid + m * p.ld_r;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = (int64_t)tn * BN + wn * 128 + i * 32 + 8 * q + 4 * g2;
                    if (n >= p.N) continue;
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    if (p.bias) {
                        const uint2 b = *reinterpret_cast<const uint2 *>(p.bias + n);
                        v[0] += bf16_lo(b.x); v[1] += bf16_hi(b.x); v[2] += bf16_lo(b.y); v[3] += bf16_hi(b.y);
                    }
                    if (EPI == H3_EPI_RESIDUAL) {
                        const float4 gv = *reinterpret_cast<const float4 *>(grow + n);
                        const uint2 rv = *reinterpret_cast<const uint2 *>(rrow + n);
                        v[0] = bf16_lo(rv.x) + gv.x * v[0];
                        v[1] = bf16_hi(rv.x) + gv.y * v[1];
                        v[2] = bf16_lo(rv.y) + gv.z * v[2];
                        v[3] = bf16_hi(rv.y) + gv.w * v[3];
                    }
                    *reinterpret_cast<uint2 *>(crow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Internal epilogue of the block's packed QKV projection, with operator group
// (2) of Sol-H3 report §3.5 ("Kernel Fusion": QK normalization with partial
// RoPE) done on the accumulators instead of as a separate HBM pass over q and
// k. A wave's 128 output columns start at a multiple of 128 and hidden is
// heads x 128, so they are exactly one head of q, k or v:
//   q, k  per row: RMSNorm over the head's 128 FP32 values (the lane pair
//         (l, l ^ 32) holds the row's two 64-value halves), times the BF16
//         gain, then the rotation of the first rot_dim channels with the
//         row's cos/sin from a table (rows with no rotation hold cos 1,
//         sin 0), rounded to BF16 once and stored in place in qkv. For k,
//         the largest squared norm of the stored BF16 rows of each head is
//         merged into kmax2[head] (an integer maximum on non-negative FP32
//         bit patterns), the bound the attention kernel's fixed softmax
//         reference needs.
//   v     stored as usual, and also written transposed into the attention's
//         V^T staging plane [heads][128][lpad] (keys permuted inside 16-key
//         groups, rows past the valid ones zero), transposed through this
//         wave's 32 KB of LDS, so attention needs no staging pass of its own.
// Args provides, besides the plain fields: q_gain, k_gain (BF16 [128]), rope
// (FP32 [rows][2][rope_half]: cos, then sin), rope_half, rope_pairing (0
// rotate-half pairs (i, i + half), 1 pairs (2i, 2i+1)), hidden, eps, vt,
// vt_lpad, kmax2.
// ---------------------------------------------------------------------------
constexpr int kEpiQkv = 4;

// Key index inside a 16-key group as the attention kernel stores V^T: bits
// 2 and 3 swapped.
__device__ __forceinline__ int vt_kperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Rotate-half RoPE on one row's values v[slot][e] (column 8 slot + 4 g2 + e):
// slot s < R16 pairs with slot s + R16 (half = 8 R16 columns apart).
template <int R16>
__device__ __forceinline__ void rope_rotate_half(float (&v)[16][4], const float *cs, int half, int g2) {
#pragma unroll
    for (int s = 0; s < R16; ++s) {
        const float4 c4 = *reinterpret_cast<const float4 *>(cs + 8 * s + 4 * g2);
        const float4 s4 = *reinterpret_cast<const float4 *>(cs + half + 8 * s + 4 * g2);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = v[s][e], b = v[s + R16][e];
            v[s][e] = a * cc[e] - b * sn[e];
            v[s + R16][e] = a * sn[e] + b * cc[e];
        }
    }
}

template <typename Args>
__device__ __forceinline__ void gemm_epilogue_qkv(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn, int wm, int wn,
                                                  int r32, int g2, uint16_t *lds_wave) {
    const int64_t n0 = (int64_t)tn * 256 + wn * 128;  // the wave's first column (wave-uniform)
    if (n0 >= p.N) return;
    const int part = (int)(n0 / p.hidden);  // 0 q, 1 k, 2 v
    const int head = (int)((n0 - (int64_t)part * p.hidden) >> 7);
    const int64_t row0 = (int64_t)tm * 256 + wm * 128;
    // bias of this lane's 64 columns (column 8 slot + 4 g2 + e)
    float bias[16][4];
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[s][e] = 0.f;
    if (p.bias) {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const uint2 b = *reinterpret_cast<const uint2 *>(p.bias + n0 + 8 * s + 4 * g2);
            bias[s][0] = bf16_lo(b.x); bias[s][1] = bf16_hi(b.x); bias[s][2] = bf16_lo(b.y); bias[s][3] = bf16_hi(b.y);
        }
    }
    if (part < 2) {
        const uint16_t *gain = part == 0 ? p.q_gain : p.k_gain;
        uint2 gw[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) gw[s] = *reinterpret_cast<const uint2 *>(gain + 8 * s + 4 * g2);
        float kmax = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t m = row0 + j * 32 + r32;
            const bool valid = m < p.M;  // the same for the lane pair (l, l ^ 32)
            float v[16][4];
            float ss = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[s][e] = acc[s >> 2][j][4 * (s & 3) + e] + bias[s][e];
                    ss += v[s][e] * v[s][e];
                }
            ss += __shfl_xor(ss, 32);
            const float inv = rsqrtf(ss * (1.0f / 128.0f) + p.eps);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float gs[4] = {bf16_lo(gw[s].x), bf16_hi(gw[s].x), bf16_lo(gw[s].y), bf16_hi(gw[s].y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) v[s][e] = v[s][e] * inv * gs[e];
            }
            if (valid && p.rope_half > 0) {
                const float *cs = p.rope + m * 2 * p.rope_half;
                const int half = p.rope_half;
                if (p.rope_pairing == 0) {
                    switch (half >> 3) {
                        case 1: rope_rotate_half<1>(v, cs, half, g2); break;
                        case 2: rope_rotate_half<2>(v, cs, half, g2); break;
                        case 3: rope_rotate_half<3>(v, cs, half, g2); break;
                        case 4: rope_rotate_half<4>(v, cs, half, g2); break;
                        case 5: rope_rotate_half<5>(v, cs, half, g2); break;
                        case 6: rope_rotate_half<6>(v, cs, half, g2); break;
                        case 7: rope_rotate_half<7>(v, cs, half, g2); break;
                        default: rope_rotate_half<8>(v, cs, half, g2); break;
                    }
                } else {
                    // pairs (2t, 2t + 1): e = (0, 1) and (2, 3) of a slot, t = 4 slot + 2 g2 + (0, 1)
#pragma unroll
                    for (int s = 0; s < 16; ++s) {
                        if (8 * s < 2 * half) {
                            const float2 c2 = *reinterpret_cast<const float2 *>(cs + 4 * s + 2 * g2);
                            const float2 s2 = *reinterpret_cast<const float2 *>(cs + half + 4 * s + 2 * g2);
                            const float cc[2] = {c2.x, c2.y}, sn[2] = {s2.x, s2.y};
#pragma unroll
                            for (int t = 0; t < 2; ++t) {
                                const float x0 = v[s][2 * t], x1 = v[s][2 * t + 1];
                                v[s][2 * t] = x0 * cc[t] - x1 * sn[t];
                                v[s][2 * t + 1] = x0 * sn[t] + x1 * cc[t];
                            }
                        }
                    }
                }
            }
            uint2 outw[16];
            float ss2 = 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                outw[s] = make_uint2(pack_bf16x2(v[s][0], v[s][1]), pack_bf16x2(v[s][2], v[s][3]));
                const float r[4] = {bf16_lo(outw[s].x), bf16_hi(outw[s].x), bf16_lo(outw[s].y), bf16_hi(outw[s].y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) ss2 = __builtin_fmaf(r[e], r[e], ss2);
            }
            ss2 += __shfl_xor(ss2, 32);
            if (valid) {
                uint16_t *crow = p.c + m * p.ldc + n0;
#pragma unroll
                for (int s = 0; s < 16; ++s) *reinterpret_cast<uint2 *>(crow + 8 * s + 4 * g2) = outw[s];
                kmax = fmaxf(kmax, ss2);
            }
        }
        if (part == 1) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, o));
            if (r32 == 0 && g2 == 0) atomicMax(p.kmax2 + head, __float_as_uint(kmax));
        }
        return;
    }
    // v: rows (valid ones) into qkv, and every row up to the V^T plane's
    // padded length into the plane, through LDS: element (channel c, key k)
    // at lds_wave[c * 128 + 8 (chunk ^ (c & 15)) + k % 8], chunk = k / 8, with
    // k already permuted inside its 16-key group.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kl = j * 32 + r32;  // key within the wave's 128 rows
        const int64_t m = row0 + kl;
        const bool valid = m < p.M;
        uint2 outw[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = valid ? acc[s >> 2][j][4 * (s & 3) + e] + bias[s][e] : 0.f;
            outw[s] = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
        if (valid) {
            uint16_t *crow = p.c + m * p.ldc + n0;
#pragma unroll
            for (int s = 0; s < 16; ++s) *reinterpret_cast<uint2 *>(crow + 8 * s + 4 * g2) = outw[s];
        }
        const int kp = vt_kperm(kl);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const uint16_t h4[4] = {(uint16_t)(outw[s].x & 0xFFFF), (uint16_t)(outw[s].x >> 16),
                                    (uint16_t)(outw[s].y & 0xFFFF), (uint16_t)(outw[s].y >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 8 * s + 4 * g2 + e;
                lds_wave[c * 128 + 8 * ((kp >> 3) ^ (c & 15)) + (kp & 7)] = h4[e];
            }
        }
    }
    // 128 channel rows x 16 chunks of 8 keys: lane reads chunk (row it*4 +
    // lane/16, chunk lane%16) and stores 16 bytes of the plane's row.
    const int lane = (int)(threadIdx.x & 63);
    uint16_t *plane = p.vt + (int64_t)head * 128 * p.vt_lpad + row0;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
        const int c = it * 4 + (lane >> 4), ch = lane & 15;
        if (row0 + 8 * ch < p.vt_lpad) {
            const uint4 val = *reinterpret_cast<const uint4 *>(lds_wave + c * 128 + 8 * (ch ^ (c & 15)));
            *reinterpret_cast<uint4 *>(plane + (int64_t)c * p.vt_lpad + 8 * ch) = val;
        }
    }
}

}  // namespace h3
