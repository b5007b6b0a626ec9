// MXFP8 MFMA GEMM for the H3 block's projections on gfx950 (Sol-H3 report,
// §3.3 "Compute Quantization", "MXFP8 GEMM computation"):
//   C = dequant(A) dequant(W)^T (+ bias), with the BF16 GEMM's epilogues
// A [M, K] and W [N, K] hold E4M3 codes, K-contiguous. Each operand carries
// one E8M0 scale per 32 consecutive k values, stored K-slab-major:
// scales[k / 128][row][4], the 4 bytes being the scales of the row's four
// 32-wide groups in that 128-wide slab. One stage's scales for a 256-row tile
// are then one contiguous kilobyte.
//
// Tiling (CDNA4): as the BF16 kernel, 256 x 256 output tile per 256-thread
// workgroup, 4 wavefronts of 128 x 128 as 4 x 4 sub-tiles of 32 x 32, the
// weight tile as the MFMA A operand. The K stage is 128 E4M3 values, again one
// whole 128-byte line per tile row, and each k-step is one
// v_mfma_scale_f32_32x32x64_f8f6f4 (64 k values, 16 passes: twice the BF16
// MFMA's flops in twice its cycles, so the stage takes the BF16 stage's time
// for twice the work).
// Operand layout of the scaled MFMA (measured on gfx950): lane l holds row
// l % 32 and 32 bytes; its bytes 0-15 belong to the row's first 32-wide k
// group of the k-step and bytes 16-31 to the second, and lane l supplies the
// scale of group l / 32. Which 16 of a group's 32 values each lane half holds
// is free as long as both operands agree: lane half h takes chunks h and 2 + h
// of the k-step's 64 bytes. The scale register's byte is chosen by the
// instruction's op-select, so each lane keeps its row's scale dword shifted
// by 8 h and op-select 2 ks picks group 2 ks + h.
// Codes go global -> LDS with direct buffer loads (16 B per lane) and scales
// with direct 4-byte loads (each wave loads 64 rows of each operand's scale
// kilobyte), double-buffered in two 66 KB stage slots; the next stage's loads
// and the next k-step's LDS reads are interleaved with the MFMAs, one barrier
// per stage.
#include "h3_device.h"
#include "h3_gemm_epilogue.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;  // BK in E4M3 values (bytes)
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 16;                   // 8 x 16 B per tile row
constexpr int kTileChunks = BM * kChunksPerRow;          // 2048 per operand tile (32 KB)
constexpr int kScaleChunks = BM * 4 / 16;                // 64: 4 scale bytes per tile row (1 KB)
constexpr int kSlotChunks = 2 * kTileChunks + 2 * kScaleChunks;  // W, A, W scales, A scales
constexpr int kSlabsPerWave = kTileChunks / 64 / 4;      // 8
constexpr int kLoadsPerStage = 2 * kSlabsPerWave + 2;    // per wave: 16 code slabs + 2 scale loads

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct MxGemmArgs {
    const uint8_t *a, *w;         // E4M3 codes
    const uint8_t *as, *ws;       // E8M0 scales, [K / 128][rows][4]
    int64_t a_srows, w_srows;     // rows of each scale array
    const uint16_t *bias;
    uint16_t *c;
    const uint16_t *resid;
    const float *gate;
    const int32_t *mod_idx;
    int64_t lda, ldw, ldc, ld_r, ld_gate;
    int64_t M, N, K;
    int32_t n_groups;
    int32_t tiles_m, tiles_n;
    int32_t group_m;
    int32_t ffn;
    uint8_t *cq;          // kEpiSwigluMx: MXFP8 output codes ...
    int64_t ld_cq;
    uint8_t *cs;          // ... and scales
    int64_t cs_rows;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ ((row >> 1) & 7)); }

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_mxfp8_kernel(MxGemmArgs p) {
    __shared__ uint4 smem[2 * kSlotChunks];

    int tm, tn;
    gemm_tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Code tiles: 32 slabs of 8 rows x 8 chunks per operand, wave w loads
    // slabs 8w .. 8w+7 (as the BF16 kernel). Scale kilobytes: wave w loads
    // tile rows 64 w .. 64 w + 63, 4 bytes per lane.
    const int64_t m_first = (int64_t)tm * BM;
    const int64_t a_rows = min<int64_t>(p.M - m_first, BM);
    const int KT = (int)(p.K / BK);
    const i32x4_t rs_a = raw_rsrc(p.a + m_first * p.lda, (a_rows - 1) * p.lda + p.K);
    i32x4_t rs_w, rs_w2;
    constexpr bool kSwiglu = EPI == H3_EPI_SWIGLU || EPI == kEpiSwigluMx;
    int64_t w_first;  // first weight row of the tile (gate block for SwiGLU)
    if (kSwiglu) {
        w_first = (int64_t)tn * (BN / 2);
        const int64_t w_rows = min<int64_t>(p.ffn - w_first, BN / 2);
        rs_w = raw_rsrc(p.w + w_first * p.ldw, (w_rows - 1) * p.ldw + p.K);
        rs_w2 = raw_rsrc(p.w + (p.ffn + w_first) * p.ldw, (w_rows - 1) * p.ldw + p.K);
    } else {
        w_first = (int64_t)tn * BN;
        const int64_t w_rows = min<int64_t>(p.N - w_first, BN);
        rs_w = raw_rsrc(p.w + w_first * p.ldw, (w_rows - 1) * p.ldw + p.K);
        rs_w2 = rs_w;
    }
    // Scale descriptors span whole arrays (rows past the tile read other
    // rows' or no scales; their outputs are never stored).
    const i32x4_t rs_as = raw_rsrc(p.as, (int64_t)KT * p.a_srows * 4);
    const i32x4_t rs_ws = raw_rsrc(p.ws, (int64_t)KT * p.w_srows * 4);
    int a_voff[kSlabsPerWave], w_voff[kSlabsPerWave];
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) {
        const int slab = 8 * wave + i;
        const int row = 8 * slab + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        a_voff[i] = (int)(row * p.lda + 16 * c);
        if (kSwiglu) {
            const int col = 16 * (slab >> 2) + 8 * (slab & 1) + (lane >> 3);
            w_voff[i] = (int)(col * p.ldw + 16 * c);
        } else {
            w_voff[i] = (int)(row * p.ldw + 16 * c);
        }
    }
    const int srow = 64 * wave + lane;  // tile row whose scale dword this lane loads
    const int as_voff = (int)((m_first + srow) * 4);
    int64_t w_srow;
    if (kSwiglu) w_srow = ((srow & 16) ? p.ffn : 0) + w_first + 16 * (srow >> 5) + (srow & 15);
    else w_srow = w_first + srow;
    const int ws_voff = (int)(w_srow * 4);
    i32x4_t rs_none = rs_a;
    rs_none.z = 0;

    const uint32_t lds_base = lds_addr(smem);
    // Direct load number d (0 .. 17) of stage kt into slot `slot`: code slab
    // 8 wave + d/2 of the A tile (d odd) or the W tile (d even) for d < 16,
    // then this wave's quarter of the W and A scale kilobytes.
    auto dma = [&](int slot, int d, int kt) {
        const bool past = kt >= KT;
        const uint32_t slot_base = lds_base + (uint32_t)(slot * kSlotChunks * 16);
        if (d < 16) {
            const int i = d >> 1, op = d & 1;
            const int slab = 8 * wave + i;
            i32x4_t r = op ? rs_a : ((kSwiglu && ((slab >> 1) & 1)) ? rs_w2 : rs_w);
            if (past) r = rs_none;
            dma_slab(r, slot_base + (uint32_t)((op * kTileChunks + 64 * slab) * 16), op ? a_voff[i] : w_voff[i],
                     kt * BK);
        } else if (d == 16) {
            // the slab offset goes into the lane offset, which the descriptor's
            // range check covers: rows past the array's end read zero
            dma_dword(past ? rs_none : rs_ws, slot_base + (uint32_t)(2 * kTileChunks * 16 + 256 * wave),
                      ws_voff + (int)((int64_t)kt * p.w_srows * 4), 0);
        } else {
            dma_dword(past ? rs_none : rs_as,
                      slot_base + (uint32_t)((2 * kTileChunks + kScaleChunks) * 16 + 256 * wave),
                      as_voff + (int)((int64_t)kt * p.a_srows * 4), 0);
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int r32 = lane & 31, g2 = lane >> 5;
    struct Ops {
        i32x8_t a[4], w[4];
    };
    struct Scales {
        int a[4], w[4];
    };
    const char *lds_bytes = reinterpret_cast<const char *>(smem);
    // Operand read r (0..7) of k-step ks of the stage in `slot`, in MFMA
    // consumption order W[0], A[0..3], W[1..3]: chunks 4 ks + g2 and
    // 4 ks + 2 + g2 of the operand row.
    auto read = [&](int slot, int ks, int r, Ops &o) {
        const uint4 *base = smem + slot * kSlotChunks;
        const bool is_a = r >= 1 && r <= 4;
        const int i = is_a ? r - 1 : (r == 0 ? 0 : r - 4);
        const int row = (is_a ? wm : wn) * 128 + i * 32 + r32;
        const uint4 *tile = base + (is_a ? kTileChunks : 0);
        const uint4 lo = tile[swz(row, 4 * ks + g2)];
        const uint4 hi = tile[swz(row, 4 * ks + 2 + g2)];
        const i32x8_t v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        if (is_a) o.a[i] = v;
        else o.w[i] = v;
    };
    // Scale dwords of the stage in `slot` for this lane's 4 W and 4 A rows,
    // shifted so that byte 2 ks is the scale of group 2 ks + g2.
    auto read_scales = [&](int slot, int r, Scales &s) {
        const char *sb = lds_bytes + (slot * kSlotChunks + 2 * kTileChunks) * 16;
        if (r < 4) {
            const int row = wn * 128 + r * 32 + r32;
            s.w[r] = (int)(*reinterpret_cast<const uint32_t *>(sb + 4 * row) >> (8 * g2));
        } else {
            const int row = wm * 128 + (r - 4) * 32 + r32;
            s.a[r - 4] = (int)(*reinterpret_cast<const uint32_t *>(sb + kScaleChunks * 16 + 4 * row) >> (8 * g2));
        }
    };
    // One k-step (16 MFMAs) of stage kt with operands `cur` and scales `sc`.
    //  ks 0: read k-step 1 of stage kt into `nxt`; issue the second 9 loads of
    //        stage kt+1 (the first 9 went out at k-step 1 of stage kt-1).
    //  ks 1: wait for stage kt+1 and for this wave's reads of stage kt,
    //        barrier, then read k-step 0 and the scales of stage kt+1 into
    //        `nxt` / `sn` and issue the first 9 loads of stage kt+2 into the
    //        slot stage kt leaves free.
    auto kstep = [&](int kt, int ks, int slot, const Ops &cur, const Scales &sc, Ops &nxt, Scales &sn) {
        if (ks == 1) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int i = t >> 2, j = t & 3;
            if (ks == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.w[i], cur.a[j], acc[i][j], 0, 0, 0,
                                                                             sc.w[i], 0, sc.a[j]);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.w[i], cur.a[j], acc[i][j], 0, 0, 2,
                                                                             sc.w[i], 2, sc.a[j]);
            if (t & 1) {
                const int d = t >> 1;
                if (ks == 1) {
                    dma(slot, d, kt + 2);
                    if (t == 15) dma(slot, 8, kt + 2);
                    read_scales(slot ^ 1, d, sn);
                } else {
                    dma(slot ^ 1, 9 + d, kt + 1);
                    if (t == 15) dma(slot ^ 1, 17, kt + 1);
                }
            } else {
                if (ks == 0) read(slot, 1, t >> 1, nxt);
                else read(slot ^ 1, 0, t >> 1, nxt);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage = [&](int kt, int slot, Ops &r0, Ops &r1, Scales &s0, Scales &s1) {
        kstep(kt, 0, slot, r0, s0, r1, s1);
        kstep(kt, 1, slot, r1, s0, r0, s1);
    };

    // Prologue: stage 0 and the first 9 loads of stage 1 in flight; stage 0's
    // k-step 0 and scales in registers.
#pragma unroll
    for (int d = 0; d < kLoadsPerStage; ++d) dma(0, d, 0);
#pragma unroll
    for (int d = 0; d < 9; ++d) dma(1, d, 1);
    Ops opa, opb;
    Scales sca, scb;
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        read(0, 0, r, opa);
        read_scales(0, r, sca);
    }
    int kt = 0;
#pragma unroll 1
    for (; kt + 2 <= KT; kt += 2) {
        stage(kt, 0, opa, opb, sca, scb);
        stage(kt + 1, 1, opa, opb, scb, sca);
    }
    if (kt < KT) stage(kt, 0, opa, opb, sca, scb);  // odd KT
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (EPI == H3_EPI_STORE || EPI == H3_EPI_RESIDUAL) {
        __syncthreads();  // every wave is done with the stage slots before they hold the epilogue's tiles
        gemm_epilogue_lds<EPI>(p, acc, tm, tn, wm, wn, lane, smem + wave * kTileChunks);
    } else {
        gemm_epilogue<EPI>(p, acc, tm, tn, wm, wn, r32, g2);
    }
}

}  // namespace

void launch_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                         const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias, uint16_t *c,
                         int64_t ldc, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                         const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
                         int32_t n_mod_groups, const int32_t *mod_idx, hipStream_t stream, uint8_t *cq,
                         int64_t ld_cq, uint8_t *cs, int64_t cs_rows) {
    if (M_valid <= 0) return;
    MxGemmArgs p;
    p.cq = cq; p.ld_cq = ld_cq; p.cs = cs; p.cs_rows = cs_rows;
    p.a = a; p.w = w; p.as = a_scales; p.ws = w_scales;
    p.a_srows = a_scale_rows; p.w_srows = N;
    p.bias = bias; p.c = c; p.resid = resid; p.gate = gate; p.mod_idx = mod_idx;
    p.lda = lda; p.ldw = ldw; p.ldc = ldc; p.ld_r = ld_r;
    p.ld_gate = n_mod_groups > 1 ? ld_gate_group : 0;
    p.M = M_valid; p.N = N; p.K = K;
    p.n_groups = n_mod_groups > 0 ? n_mod_groups : 1;
    p.ffn = (int32_t)(N / 2);
    p.tiles_m = (int32_t)((M_valid + BM - 1) / BM);
    const bool swiglu = epilogue == H3_EPI_SWIGLU || epilogue == kEpiSwigluMx;
    p.tiles_n = swiglu ? (int32_t)((N / 2 + BN / 2 - 1) / (BN / 2)) : (int32_t)((N + BN - 1) / BN);
    p.group_m = p.tiles_n >= 128 ? 8 : 2;
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    switch (epilogue) {
        case H3_EPI_RESIDUAL: gemm_mxfp8_kernel<H3_EPI_RESIDUAL><<<grid, kThreads, 0, stream>>>(p); break;
        case H3_EPI_SWIGLU: gemm_mxfp8_kernel<H3_EPI_SWIGLU><<<grid, kThreads, 0, stream>>>(p); break;
        case kEpiSwigluMx: gemm_mxfp8_kernel<kEpiSwigluMx><<<grid, kThreads, 0, stream>>>(p); break;
        default: gemm_mxfp8_kernel<H3_EPI_STORE><<<grid, kThreads, 0, stream>>>(p); break;
    }
}

}  // namespace h3

using namespace h3;

extern "C" int h3_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                               const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias,
                               uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                               int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                               int64_t ld_gate_group, int32_t n_mod_groups, const int32_t *mod_idx, void *stream) {
    int s = h3_check_linear_mxfp8(a, lda, a_scales, a_scale_rows, w, ldw, w_scales, bias, c, ldc, M_buf, M_valid, N,
                                  K, epilogue, resid, ld_r, gate, ld_gate_group, n_mod_groups);
    if (s != H3_OK || M_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    launch_linear_mxfp8(a, lda, a_scales, a_scale_rows, w, ldw, w_scales, bias, c, ldc, M_valid, N, K, epilogue,
                        resid, ld_r, gate, ld_gate_group, n_mod_groups, mod_idx, st);
    launch_zero_rows(c, ldc, epilogue == H3_EPI_SWIGLU ? N / 2 : N, M_valid, M_buf, st);
    return launch_status();
}
