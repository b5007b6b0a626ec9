// BF16 MFMA GEMM for the H3 block's projections on gfx950:
//   C = A W^T (+ bias), A [M, K] activations, W [N, K] weights, both K-contiguous.
// The packed QKV projection (Sol-H3 report, §3.2 "Optimized attention
// collectives": packed QKV storage), the output projection and the SwiGLU FFN
// (§3.5 "Kernel Fusion") are all this shape. Two of §3.5's operator groups run
// in the epilogue instead of as separate HBM passes:
//   H3_EPI_RESIDUAL  group (1)'s residual addition with indexed gating;
//   H3_EPI_SWIGLU    group (3): the gate and up halves of W are interleaved in
//                    16-row blocks inside a tile, so silu(gate) * up is formed
//                    from two accumulators held by the same lane and the
//                    [M, 2F] intermediate never reaches HBM.
//
// Tiling (CDNA4): 256 x 256 output tile per 256-thread workgroup, 4 wavefronts
// of 128 x 128, K step 64, v_mfma_f32_32x32x16_bf16. The weight tile is the
// MFMA A operand and the activation tile the B operand, so each lane's
// accumulator holds groups of 4 consecutive output columns of one row
// (8-byte stores).
// LDS holds two stages of both tiles (128 KB) with a 16-byte-chunk XOR swizzle
// (chunk c of row r at c ^ (r & 7)): conflict-free 128-bit reads and writes.
// Tiles are ordered so each XCD (workgroups are dealt round-robin over 8 XCDs)
// walks a contiguous range of a grouped tile order, keeping the operand
// K-slices its 32 CUs share in that XCD's L2.
#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 8;                    // 8 x 16 B
constexpr int kTileChunks = BM * kChunksPerRow;           // 2048 per operand tile
constexpr int kLoadsPerThread = kTileChunks / kThreads;   // 8
constexpr int kGroupM = 8;

struct GemmArgs {
    const uint16_t *a;
    const uint16_t *w;
    const uint16_t *bias;
    uint16_t *c;
    const uint16_t *resid;
    const float *gate;
    const int32_t *mod_idx;
    int64_t lda, ldw, ldc, ld_r, ld_gate;
    int64_t M, N, K;      // M valid rows; N weight rows; K reduction
    int32_t n_groups;
    int32_t tiles_m, tiles_n;
    int32_t ffn;          // SwiGLU output width
};

// Raw buffer descriptor over `bytes` bytes from `base` (clamped to 4 GiB);
// loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    // Every descriptor is wave-uniform by construction; readfirstlane keeps it
    // in scalar registers even where the index arithmetic ran on the VALU.
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int32_t n = __builtin_amdgcn_readfirstlane(bytes >= 0xFFFFFFFFll ? (int32_t)0xFFFFFFFF : (int32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ (row & 7)); }

// Map a linear workgroup id to (tile_m, tile_n): XCD-contiguous ranges of a
// grouped (kGroupM tile-rows at a time) order.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int T = tiles_m * tiles_n;
    const int q = T / 8, rr = T % 8;
    const int xcd = bid % 8, local = bid / 8;
    const int lin = xcd < rr ? xcd * (q + 1) + local : rr * (q + 1) + (xcd - rr) * q + local;
    const int per_group = kGroupM * tiles_n;
    const int group = lin / per_group;
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_group = lin - group * per_group;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs p) {
    __shared__ uint4 lds[2][2][kTileChunks];  // [stage][0 = W, 1 = A]

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;

    // Thread t loads 16-byte chunk c = t & 7 of tile rows r0 + 32 j (j < 8),
    // r0 = t >> 3, through buffer loads: a wave-uniform resource descriptor
    // spans the tile's valid rows, so rows past M (or N) read as zero without a
    // branch, and the K offset and row step travel in a scalar offset. The
    // SwiGLU weight tile interleaves 16-row blocks of the gate and up halves:
    // tile row r0 + 32 j is gate (waves 0-1, r0 < 16) or up (waves 2-3) column
    // tn * 128 + 16 j + (r0 & 15).
    const int r0 = t >> 3, c8 = 8 * (t & 7);
    const int64_t m_first = (int64_t)tm * BM;
    const int64_t a_rows = min<int64_t>(p.M - m_first, BM);
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a + m_first * p.lda, ((a_rows - 1) * p.lda + p.K) * 2);
    const int voff_a = (int)((r0 * p.lda + c8) * 2);
    const int a_row_step = (int)(32 * p.lda * 2);
    __amdgpu_buffer_rsrc_t rs_w;
    int voff_w, w_row_step;
    if (EPI == H3_EPI_SWIGLU) {
        const int64_t col_first = (int64_t)tn * (BN / 2);
        const int64_t w_rows = min<int64_t>(p.ffn - col_first, BN / 2);
        const int64_t half = wave >> 1;
        rs_w = make_rsrc(p.w + (half * p.ffn + col_first) * p.ldw, ((w_rows - 1) * p.ldw + p.K) * 2);
        voff_w = (int)(((r0 & 15) * p.ldw + c8) * 2);
        w_row_step = (int)(16 * p.ldw * 2);
    } else {
        const int64_t n_first = (int64_t)tn * BN;
        const int64_t w_rows = min<int64_t>(p.N - n_first, BN);
        rs_w = make_rsrc(p.w + n_first * p.ldw, ((w_rows - 1) * p.ldw + p.K) * 2);
        voff_w = (int)((r0 * p.ldw + c8) * 2);
        w_row_step = (int)(32 * p.ldw * 2);
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = (int)(p.K / BK);
    uint4 ra[kLoadsPerThread], rw[kLoadsPerThread];
    auto gload = [&](int kt) {
        const int k0b = kt * BK * 2;
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            ra[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_a, voff_a, k0b + j * a_row_step, 0));
            rw[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, voff_w, k0b + j * w_row_step, 0));
        }
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int j = 0; j < kLoadsPerThread; ++j) {
            const int pos = swz(r0 + 32 * j, t & 7);
            lds[stage][0][pos] = rw[j];
            lds[stage][1][pos] = ra[j];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    const int r32 = lane & 31, g2 = lane >> 5;
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        gload(kt + 1);  // the last prefetch reads a harmless in-descriptor tile
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMA work
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8_t aop[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                aop[j] = __builtin_bit_cast(bf16x8_t, lds[st][1][swz(wm * 128 + j * 32 + r32, ks * 2 + g2)]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8_t wop = __builtin_bit_cast(bf16x8_t, lds[st][0][swz(wn * 128 + i * 32 + r32, ks * 2 + g2)]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop, aop[j], acc[i][j], 0, 0, 0);
            }
        }
        lstore(st ^ 1);
        __syncthreads();
    }

    // Epilogue: in each 32 x 32 sub-tile the lane holds row m = lane & 31 and,
    // for register group q (0..3), the 4 columns 8 q + 4 (lane >> 5) + (0..3).
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = (int64_t)tm * BM + wm * 128 + j * 32 + r32;
        if (m >= p.M) continue;
        uint16_t *crow = p.c + m * p.ldc;
        if (EPI == H3_EPI_SWIGLU) {
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

}  // namespace

void launch_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                   uint16_t *c, int64_t ldc, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                   const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
                   int32_t n_mod_groups, const int32_t *mod_idx, hipStream_t stream) {
    if (M_valid <= 0) return;
    GemmArgs p;
    p.a = a; p.w = w; p.bias = bias; p.c = c; p.resid = resid; p.gate = gate; p.mod_idx = mod_idx;
    p.lda = lda; p.ldw = ldw; p.ldc = ldc; p.ld_r = ld_r;
    p.ld_gate = n_mod_groups > 1 ? ld_gate_group : 0;
    p.M = M_valid; p.N = N; p.K = K;
    p.n_groups = n_mod_groups > 0 ? n_mod_groups : 1;
    p.ffn = (int32_t)(N / 2);
    p.tiles_m = (int32_t)((M_valid + BM - 1) / BM);
    p.tiles_n = epilogue == H3_EPI_SWIGLU ? (int32_t)((N / 2 + BN / 2 - 1) / (BN / 2)) : (int32_t)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    switch (epilogue) {
        case H3_EPI_RESIDUAL: gemm_bf16_kernel<H3_EPI_RESIDUAL><<<grid, kThreads, 0, stream>>>(p); break;
        case H3_EPI_SWIGLU: gemm_bf16_kernel<H3_EPI_SWIGLU><<<grid, kThreads, 0, stream>>>(p); break;
        default: gemm_bf16_kernel<H3_EPI_STORE><<<grid, kThreads, 0, stream>>>(p); break;
    }
}

}  // namespace h3

using namespace h3;

extern "C" int h3_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                         uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                         int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                         int64_t ld_gate_group, int32_t n_mod_groups, const int32_t *mod_idx, void *stream) {
    int s = h3_check_linear(a, lda, w, ldw, c, ldc, M_buf, M_valid, N, K, epilogue, resid, ld_r, gate,
                            n_mod_groups);
    if (s != H3_OK || M_buf == 0) return s;
    if (bias && (reinterpret_cast<uintptr_t>(bias) & 15u)) return H3_ERR_ALIGN;
    if (epilogue == H3_EPI_RESIDUAL && n_mod_groups > 1 && (ld_gate_group % 4) != 0) return H3_ERR_ALIGN;
    if ((s = device_check()) != H3_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    launch_linear(a, lda, w, ldw, bias, c, ldc, M_valid, N, K, epilogue, resid, ld_r, gate, ld_gate_group,
                  n_mod_groups, mod_idx, st);
    launch_zero_rows(c, ldc, epilogue == H3_EPI_SWIGLU ? N / 2 : N, M_valid, M_buf, st);
    return launch_status();
}
