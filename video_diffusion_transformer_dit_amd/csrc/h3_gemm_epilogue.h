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
// gemm_epilogue_rows handles the wave's 32-row block J, sub-tiles acc[i][J]
// (the other entries of acc are not read).
template <int EPI, int J, typename Args>
__device__ __forceinline__ void gemm_epilogue_rows(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn, int wm,
                                                   int wn, int r32, int g2) {
    constexpr int BM = 256, BN = 256;
    constexpr int j = J;
    {
        const int64_t m = (int64_t)tm * BM + wm * 128 + j * 32 + r32;
        if (m >= p.M) return;
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
                            o[ii][q][e] = silu(zg) * (acc[i][j][4 * (q + 2) + e] + ub[e]);
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
                        o[e] = silu(zg) * (acc[i][j][4 * (q + 2) + e] + ub[e]);
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
            // Every load of the row first, then the stores: a load after a
            // store that might alias it would wait out a memory latency. (The
            // GEMM kernels' own store / residual epilogue is gemm_epilogue_lds;
            // this path serves the stream-K fix-up, which has registers to
            // spare.)
            uint2 bv[4][4], rv[4][4];
            float4 gv[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = (int64_t)tn * BN + wn * 128 + i * 32 + 8 * q + 4 * g2;
                    if (n >= p.N) continue;
                    if (p.bias) bv[i][q] = *reinterpret_cast<const uint2 *>(p.bias + n);
                    if (EPI == H3_EPI_RESIDUAL) {
                        gv[i][q] = *reinterpret_cast<const float4 *>(grow + n);
                        rv[i][q] = *reinterpret_cast<const uint2 *>(rrow + n);
                    }
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = (int64_t)tn * BN + wn * 128 + i * 32 + 8 * q + 4 * g2;
                    if (n >= p.N) continue;
                    float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    if (p.bias) {
                        const uint2 b = bv[i][q];
                        v[0] += bf16_lo(b.x); v[1] += bf16_hi(b.x); v[2] += bf16_lo(b.y); v[3] += bf16_hi(b.y);
                    }
                    if (EPI == H3_EPI_RESIDUAL) {
                        const float4 g4 = gv[i][q];
                        const uint2 r2 = rv[i][q];
                        v[0] = bf16_lo(r2.x) + g4.x * v[0];
                        v[1] = bf16_hi(r2.x) + g4.y * v[1];
                        v[2] = bf16_lo(r2.y) + g4.z * v[2];
                        v[3] = bf16_hi(r2.y) + g4.w * v[3];
                    }
                    *reinterpret_cast<uint2 *>(crow + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        }
    }
}

// Gated-residual epilogue through LDS: the wave's residual block (128 rows x
// 128 columns, BF16, [128 rows][16 chunks of 8], chunk c of row r at
// c ^ (r & 15)) streams into its 32 KB of LDS with direct loads, one latency
// for the whole block; each lane then reads its 4-column pieces there, forms
// resid + gate * (acc + bias), writes the BF16 result back in place, and the
// block leaves row by row with 16-byte stores. The caller has made the LDS
// free (barrier); everything after is wave-local.
template <typename Args>
__device__ __forceinline__ void gemm_epilogue_residual_lds(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn,
                                                           int wm, int wn, int lane, uint4 *lw) {
    constexpr int BM = 256, BN = 256;
    const int r32 = lane & 31, g2 = lane >> 5;
    const int64_t row0 = (int64_t)tm * BM + wm * 128;
    const int64_t col0 = (int64_t)tn * BN + wn * 128;
    const int64_t rows = min<int64_t>(p.M - row0, 128);
    if (rows <= 0 || col0 >= p.N) return;
    const int64_t cols = min<int64_t>(p.N - col0, 128);
    // residual block -> LDS: slab s (1 KB) is rows 4 s .. 4 s + 3; lane i
    // lands at physical chunk i & 15 of row 4 s + i / 16 and so loads that
    // row's logical chunk (i & 15) ^ (row & 15). Rows past M read zero.
    const i32x4_t rs = raw_rsrc(p.resid + row0 * p.ld_r + col0, ((rows - 1) * p.ld_r + cols) * 2);
    const uint32_t lds_w = lds_addr(lw);
#pragma unroll
    for (int sl = 0; sl < 32; ++sl) {
        const int row = 4 * sl + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);
        dma_slab(rs, lds_w + (uint32_t)(sl * 1024), (int)((row * p.ld_r + 8 * c) * 2), 0);
    }
    // per-column operands, the same for every row unless rows pick gate groups
    const bool gate_per_row = p.mod_idx != nullptr;
    float4 gv[4][4];
    uint2 bv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = col0 + i * 32 + 8 * q + 4 * g2;
            gv[i][q] = make_float4(0.f, 0.f, 0.f, 0.f);
            bv[i][q] = make_uint2(0u, 0u);
            if (n < p.N) {
                if (!gate_per_row) gv[i][q] = *reinterpret_cast<const float4 *>(p.gate + n);
                if (p.bias) bv[i][q] = *reinterpret_cast<const uint2 *>(p.bias + n);
            }
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the residual block is in LDS
    uint2 *lh = reinterpret_cast<uint2 *>(lw);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = j * 32 + r32;
        const float *grow = p.gate;
        if (gate_per_row && row < rows) {
            const int g = min(max(p.mod_idx[row0 + row], 0), p.n_groups - 1);
            grow = p.gate + (int64_t)g * p.ld_gate;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = col0 + i * 32 + 8 * q + 4 * g2;
                const int at = (row * 16 + ((4 * i + q) ^ (row & 15))) * 2 + g2;
                const uint2 r2 = lh[at];
                float4 g4 = gv[i][q];
                if (gate_per_row && row < rows && n < p.N) g4 = *reinterpret_cast<const float4 *>(grow + n);
                const uint2 b = bv[i][q];
                const float v0 = acc[i][j][4 * q] + bf16_lo(b.x), v1 = acc[i][j][4 * q + 1] + bf16_hi(b.x);
                const float v2 = acc[i][j][4 * q + 2] + bf16_lo(b.y), v3 = acc[i][j][4 * q + 3] + bf16_hi(b.y);
                lh[at] = make_uint2(pack_bf16x2(bf16_lo(r2.x) + g4.x * v0, bf16_hi(r2.x) + g4.y * v1),
                                    pack_bf16x2(bf16_lo(r2.y) + g4.z * v2, bf16_hi(r2.y) + g4.w * v3));
            }
    }
    const int c = lane & 15;
#pragma unroll
    for (int it = 0; it < 32; ++it) {
        const int row = it * 4 + (lane >> 4);
        const uint4 val = lw[row * 16 + (c ^ (row & 15))];
        if (row < rows && 8 * c < cols) *reinterpret_cast<uint4 *>(p.c + (row0 + row) * p.ldc + col0 + 8 * c) = val;
    }
}

// Epilogue through LDS. In the MFMA register layout a lane holds 4 columns of
// one row per register group, so a wave's global accesses would touch 32 rows
// in 8- or 16-byte pieces. Instead each wave writes its 128 x 128 results to
// its own 32 KB of the (now idle) stage ring and reads them back row by row,
// so every global load and store is 16 bytes per lane along a row (whole
// 128-byte lines per 8 lanes). Same arithmetic per element as gemm_epilogue.
// lw: the wave's 32 KB of LDS, free of other use; Args as for gemm_epilogue.
// The FP32 accumulators go half the wave's rows at a time ([64 rows][32
// chunks of 4 floats], chunk k of row r at k ^ (r & 15)); a lane then takes
// 8 columns of one row, 4 rows per step. Store and gated-residual epilogues
// (measured 2-4% faster on the BF16 projections that use them); the SwiGLU tile,
// half as wide at the output, measured the same either way and keeps the
// register-layout epilogue.
template <int EPI, typename Args>
__device__ __forceinline__ void gemm_epilogue_lds(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn, int wm,
                                                  int wn, int lane, uint4 *lw) {
    if constexpr (EPI == H3_EPI_RESIDUAL) {
        gemm_epilogue_residual_lds(p, acc, tm, tn, wm, wn, lane, lw);
        return;
    }
    constexpr int BM = 256, BN = 256;
    const int r32 = lane & 31, g2 = lane >> 5;
    const int64_t row0 = (int64_t)tm * BM + wm * 128;
    const int c8 = lane & 15;
    const int64_t n = (int64_t)tn * BN + wn * 128 + 8 * c8;
    const bool col_ok = n < p.N;
    float bias8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (p.bias && col_ok) unpack8(*reinterpret_cast<const uint4 *>(p.bias + n), bias8);
    // one gate row for every row unless the rows pick modulation groups
    const bool gate_per_row = EPI == H3_EPI_RESIDUAL && p.mod_idx != nullptr;
    float gate8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (EPI == H3_EPI_RESIDUAL && !gate_per_row && col_ok) {
        const float4 g0 = *reinterpret_cast<const float4 *>(p.gate + n);
        const float4 g1 = *reinterpret_cast<const float4 *>(p.gate + n + 4);
        gate8[0] = g0.x; gate8[1] = g0.y; gate8[2] = g0.z; gate8[3] = g0.w;
        gate8[4] = g1.x; gate8[5] = g1.y; gate8[6] = g1.z; gate8[7] = g1.w;
    }
    float4 *lf = reinterpret_cast<float4 *>(lw);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * h + jj;
            const int row = jj * 32 + r32;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int chunk = 8 * i + 2 * q + g2;
                    lf[row * 32 + (chunk ^ (row & 15))] = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                                      acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                }
        }
        // the residual rows of this half first: loads issued after the
        // stores below would each wait out a latency (possible aliasing)
        uint4 rv[16];
        if (EPI == H3_EPI_RESIDUAL) {
#pragma unroll
            for (int it = 0; it < 16; ++it) {
                const int64_t m = row0 + 64 * h + it * 4 + (lane >> 4);
                if (m < p.M && col_ok) rv[it] = *reinterpret_cast<const uint4 *>(p.resid + m * p.ld_r + n);
            }
        }
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = it * 4 + (lane >> 4);
            const int64_t m = row0 + 64 * h + row;
            const float4 a = lf[row * 32 + ((2 * c8) ^ (row & 15))];
            const float4 b = lf[row * 32 + ((2 * c8 + 1) ^ (row & 15))];
            if (m >= p.M || !col_ok) continue;
            float v[8] = {a.x + bias8[0], a.y + bias8[1], a.z + bias8[2], a.w + bias8[3],
                          b.x + bias8[4], b.y + bias8[5], b.z + bias8[6], b.w + bias8[7]};
            if (EPI == H3_EPI_RESIDUAL) {
                float g[8];
                if (gate_per_row) {
                    const int grp = min(max(p.mod_idx[m], 0), p.n_groups - 1);
                    const float *gr = p.gate + (int64_t)grp * p.ld_gate + n;
                    const float4 g0 = *reinterpret_cast<const float4 *>(gr);
                    const float4 g1 = *reinterpret_cast<const float4 *>(gr + 4);
                    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
                    g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) g[e] = gate8[e];
                }
                float r[8];
                unpack8(rv[it], r);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = r[e] + g[e] * v[e];
            }
            *reinterpret_cast<uint4 *>(p.c + m * p.ldc + n) = pack8(v);
        }
    }
}

// The whole wave's 128 x 128: acc[i][j] is sub-tile (i, j).
template <int EPI, typename Args>
__device__ __forceinline__ void gemm_epilogue(const Args &p, f32x16_t (&acc)[4][4], int tm, int tn, int wm, int wn,
                                              int r32, int g2) {
    gemm_epilogue_rows<EPI, 0>(p, acc, tm, tn, wm, wn, r32, g2);
    gemm_epilogue_rows<EPI, 1>(p, acc, tm, tn, wm, wn, r32, g2);
    gemm_epilogue_rows<EPI, 2>(p, acc, tm, tn, wm, wn, r32, g2);
    gemm_epilogue_rows<EPI, 3>(p, acc, tm, tn, wm, wn, r32, g2);
}

}  // namespace h3
