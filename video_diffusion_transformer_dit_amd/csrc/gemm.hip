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
// of 128 x 128, K step 32, v_mfma_f32_32x32x16_bf16. The weight tile is the
// MFMA A operand and the activation tile the B operand, so each lane's
// accumulator holds groups of 4 consecutive output columns of one row
// (8-byte stores).
// Operand tiles go global -> LDS directly (buffer loads with the LDS bit, no
// register staging) through a 4-stage ring of 2 x 16 KB slots (128 KB): three
// K steps are in flight while the fourth is consumed, with explicit vmcnt
// waits, so a step waits only for its own stage. A 16-byte-chunk XOR swizzle
// keeps the 128-bit LDS reads conflict-free.
// Tiles are ordered so each XCD (workgroups are dealt round-robin over 8 XCDs)
// walks a contiguous range of a grouped tile order, keeping the operand
// K-slices its 32 CUs share in that XCD's L2.
#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int kThreads = 256;
constexpr int kStages = 4;                                // LDS ring depth
constexpr int kChunksPerRow = BK / 8;                     // 4 x 16 B per tile row
constexpr int kTileChunks = BM * kChunksPerRow;           // 1024 per operand tile (16 KB)
constexpr int kSlabsPerWave = kTileChunks / 64 / 4;       // 1 KB slabs per wave per operand: 4
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

// LDS operand tile: row r holds 4 chunks of 16 B (32 k values); chunk c of row
// r is stored at c ^ ((r >> 2) & 3), so the 8 lanes an LDS cycle serves (rows
// r..r+7, one chunk) hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ ((row >> 2) & 3)); }

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
    // LDS ring: kStages slots of [W tile, A tile], 16 KB each (128 KB).
    __shared__ uint4 smem[kStages * 2 * kTileChunks];

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;

    // Operand tiles stream straight into LDS (gfx950 buffer loads with the LDS
    // bit: lane i's 16 bytes land at slab + 16 i). A 16 KB operand tile is 16
    // slabs of 16 rows x 4 chunks; wave w loads slabs 4w .. 4w+3 of both
    // operands. Lane i of a slab holds row 16 s + i/4 and physical chunk i%4,
    // i.e. logical chunk (i%4) ^ ((row >> 2) & 3). A wave-uniform buffer
    // descriptor spans the tile's valid rows: rows past M (or N) read as zero.
    // The SwiGLU weight tile interleaves 16-row blocks of the gate and up
    // halves: tile row r is gate (r & 16 == 0) or up column tn*128 + 16 (r/32) + r%16.
    const int64_t m_first = (int64_t)tm * BM;
    const int64_t a_rows = min<int64_t>(p.M - m_first, BM);
    const i32x4_t rs_a = raw_rsrc(p.a + m_first * p.lda, ((a_rows - 1) * p.lda + p.K) * 2);
    i32x4_t rs_w, rs_w2;
    if (EPI == H3_EPI_SWIGLU) {
        const int64_t col_first = (int64_t)tn * (BN / 2);
        const int64_t w_rows = min<int64_t>(p.ffn - col_first, BN / 2);
        rs_w = raw_rsrc(p.w + col_first * p.ldw, ((w_rows - 1) * p.ldw + p.K) * 2);
        rs_w2 = raw_rsrc(p.w + (p.ffn + col_first) * p.ldw, ((w_rows - 1) * p.ldw + p.K) * 2);
    } else {
        const int64_t n_first = (int64_t)tn * BN;
        const int64_t w_rows = min<int64_t>(p.N - n_first, BN);
        rs_w = raw_rsrc(p.w + n_first * p.ldw, ((w_rows - 1) * p.ldw + p.K) * 2);
        rs_w2 = rs_w;
    }
    int a_voff[kSlabsPerWave], w_voff[kSlabsPerWave];
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) {
        const int slab = 4 * wave + i;
        const int row = 16 * slab + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 2) & 3);
        a_voff[i] = (int)((row * p.lda + 8 * c) * 2);
        if (EPI == H3_EPI_SWIGLU) {
            // slab rows are all gate (slab even) or all up (slab odd)
            const int col = 16 * (slab >> 1) + (lane >> 2);
            w_voff[i] = (int)((col * p.ldw + 8 * c) * 2);
        } else {
            w_voff[i] = (int)((row * p.ldw + 8 * c) * 2);
        }
    }
    // Stages past the end of K load through a zero-length descriptor: the
    // loads return zero without touching memory, so every step issues the
    // same 8 loads and the vmcnt arithmetic below is constant.
    i32x4_t rs_none = rs_a;
    rs_none.z = 0;
    // LDS byte address of this wave's first slab of slot 0's W tile.
    const uint32_t lds_wave = lds_addr(smem) + (uint32_t)(4 * wave * 64 * 16);
    // Direct load number d (0..7) of stage kt into ring slot `slot`: slab
    // 4 wave + d/2 of the A tile (d odd) or the W tile (d even).
    auto dma = [&](int slot, int d, int kt, bool live) {
        const int i = d >> 1, op = (d & 1) ? 1 : 0;
        const int slab = 4 * wave + i;
        i32x4_t r = op ? rs_a : ((EPI == H3_EPI_SWIGLU && (slab & 1)) ? rs_w2 : rs_w);
        if (!live) r = rs_none;
        const uint32_t m0 = lds_wave + (uint32_t)(((slot * 2 + op) * kTileChunks + 64 * i) * 16);
        dma_slab(r, m0, op ? a_voff[i] : w_voff[i], kt * BK * 2);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = (int)(p.K / BK);
    const int r32 = lane & 31, g2 = lane >> 5;
    // This wave's MFMA operands of one stage: [ks][sub-tile] for A and W.
    struct Ops {
        bf16x8_t a[2][4], w[2][4];
    };
    // LDS read number r (0..15) of a stage, in the order the MFMAs consume
    // the operands: per half ks, W[0], A[0..3], W[1..3].
    auto read = [&](int slot, int r, Ops &o) {
        const int ks = r >> 3, q = r & 7;
        const uint4 *base = smem + slot * 2 * kTileChunks;
        if (q >= 1 && q <= 4)
            o.a[ks][q - 1] = __builtin_bit_cast(bf16x8_t, base[kTileChunks + swz(wm * 128 + (q - 1) * 32 + r32, ks * 2 + g2)]);
        else {
            const int i = q == 0 ? 0 : q - 4;
            o.w[ks][i] = __builtin_bit_cast(bf16x8_t, base[swz(wn * 128 + i * 32 + r32, ks * 2 + g2)]);
        }
    };
    // One ring step. On entry `cur` holds stage kt's operands (read from LDS
    // during the previous step) and stages kt+1, kt+2 are in flight. Wait for
    // stage kt+1 (8 loads per stage per wave: vmcnt 8 leaves kt+2 pending),
    // barrier (every wave has then also consumed the LDS slot of stage kt-1),
    // then run stage kt's 32 MFMAs on `cur` with the refill of that slot
    // (stage kt+3, one direct load every 4th MFMA) and the 16 LDS reads of
    // stage kt+1 into `nxt` in between, in a fixed order, so the load issue
    // never leaves the matrix pipe idle. Raw barrier: __syncthreads()'s
    // fences would wait for every outstanding load. When kt+1 == KT the slot
    // read is stale and the values unused.
    auto step = [&](int kt, int slot_next, int slot_refill, const Ops &cur, Ops &nxt) {
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const bool live = kt + 3 < KT;
        int r = 0;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            const int ks = t >> 4, i = (t >> 2) & 3, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.w[ks][i], cur.a[ks][j], acc[i][j], 0, 0, 0);
            if ((t & 3) == 0) dma(slot_refill, t >> 2, kt + 3, live);
            else if (r < 16) read(slot_next, r++, nxt);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: stages 0..2 in flight, stage 0's operands in registers.
#pragma unroll
    for (int st = 0; st < 3; ++st)
#pragma unroll
        for (int d = 0; d < 8; ++d) dma(st, d, st, st < KT);
    Ops opa, opb;
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 16; ++r) read(0, r, opa);
    int kt = 0;
#pragma unroll 1
    for (; kt + 4 <= KT; kt += 4) {
        step(kt + 0, 1, 3, opa, opb);
        step(kt + 1, 2, 0, opb, opa);
        step(kt + 2, 3, 1, opa, opb);
        step(kt + 3, 0, 2, opb, opa);
    }
    if (kt < KT) step(kt, 1, 3, opa, opb);  // remainder: KT % 4 steps
    if (kt + 1 < KT) step(kt + 1, 2, 0, opb, opa);
    if (kt + 2 < KT) step(kt + 2, 3, 1, opa, opb);
    // Drain the loads still in flight (stages past K) before the workgroup
    // can end.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
