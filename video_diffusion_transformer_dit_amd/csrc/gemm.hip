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
// of 128 x 128, K stage 64, v_mfma_f32_32x32x16_bf16. The weight tile is the
// MFMA A operand and the activation tile the B operand, so each lane's
// accumulator holds groups of 4 consecutive output columns of one row
// (8-byte stores).
// Operand tiles go global -> LDS directly (buffer loads with the LDS bit, no
// register staging) into a ring of five 32 KB operand tiles, so the weight
// tile of a stage streams in two stages ahead and the activation tile one
// stage ahead. A stage is 64 k values, i.e. one whole 128-byte line per tile
// row, so no line is fetched twice into the CU. The loads and the next
// k-step's LDS operand reads are interleaved with the current k-step's MFMAs,
// with one barrier per stage. A 16-byte-chunk XOR swizzle keeps the 128-bit
// LDS reads conflict-free. The store and gated-residual epilogues pass the
// accumulators through the idle ring so that global accesses run along rows.
// Tiles are ordered so each XCD (workgroups are dealt round-robin over 8 XCDs)
// walks a contiguous range of a grouped tile order, keeping the operand
// K-slices its 32 CUs share in that XCD's L2.
#include "h3_device.h"
#include "h3_gemm_epilogue.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 8;                     // 8 x 16 B per tile row: one 128 B line
constexpr int kTileChunks = BM * kChunksPerRow;           // 2048 per operand tile (32 KB)
constexpr int kSlabsPerWave = kTileChunks / 64 / 4;       // 1 KB slabs per wave per operand: 8

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
    int32_t group_m;      // tile rows per group of the tile order
    int32_t ffn;          // SwiGLU output width
    // Stream-K tail: workgroups [0, dp_tiles) each own a whole tile; the last
    // sk_tiles tiles of the order are cut into sk_groups equal ranges of
    // (tile, K stage) units, whose FP32 partial sums go to `part` (two
    // 256 x 256 slots per range) for the fix-up pass.
    int32_t dp_tiles, sk_tiles, sk_groups;
    float *part;
    // Tile dealing: on each XCD, the first static_tickets workgroups take the
    // tile of their index; the later ones draw one from the XCD's counter in
    // `queue` (queue == nullptr: none draw).
    int32_t *queue;
    int32_t static_tickets;
};

// LDS operand tile: row r holds 8 chunks of 16 B (64 k values); chunk c of
// row r is stored at c ^ ((r >> 1) & 7). A 128-bit LDS read serves 16 lanes
// (rows r..r+15, one chunk) per cycle: the 8 even and the 8 odd rows each
// see 8 distinct chunk positions, so the 16 reads hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ ((row >> 1) & 7)); }

// One output tile (tm, tn) over the K stages [k0, k1): the whole tile with
// its epilogue, or (PARTIAL) a range of its stages whose FP32 partial sums go
// to `part` (stream-K tail). smem: the 160 KB ring of operand tiles.
template <int EPI, bool PARTIAL>
__device__ __forceinline__ void gemm_tile(const GemmArgs &p, uint4 *smem, int tm, int tn, int k0, int k1,
                                          float *part) {
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;

    // Operand tiles stream straight into LDS (gfx950 buffer loads with the LDS
    // bit: lane i's 16 bytes land at slab + 16 i). A 32 KB operand tile is 32
    // slabs of 8 rows x 8 chunks, so each load instruction covers whole 128 B
    // lines of 8 rows; wave w loads slabs 8w .. 8w+7 of both operands. Lane i
    // of a slab holds row 8 s + i/8 and physical chunk i%8, i.e. logical chunk
    // (i%8) ^ ((row >> 1) & 7). A wave-uniform buffer descriptor spans the
    // tile's valid rows: rows past M (or N) read as zero.
    // The SwiGLU weight tile interleaves 16-row blocks of the gate and up
    // halves: tile row r is gate ((r & 16) == 0) or up, of output column
    // tn*128 + 16 (r/32) + r%16.
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
        const int slab = 8 * wave + i;
        const int row = 8 * slab + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        a_voff[i] = (int)((row * p.lda + 8 * c) * 2);
        if (EPI == H3_EPI_SWIGLU) {
            // a slab's 8 rows lie in one 16-row gate (slab/2 even) or up block
            const int col = 16 * (slab >> 2) + 8 * (slab & 1) + (lane >> 3);
            w_voff[i] = (int)((col * p.ldw + 8 * c) * 2);
        } else {
            w_voff[i] = (int)((row * p.ldw + 8 * c) * 2);
        }
    }
    // Stages past the end of the range load through a zero-length descriptor:
    // the loads return zero without touching memory, so every stage issues
    // the same 16 loads and the vmcnt arithmetic below is constant.
    i32x4_t rs_none = rs_a;
    rs_none.z = 0;
    // LDS holds a ring of 5 operand tiles of 32 KB ("halves" of a stage).
    // Stage s (counted from k0) keeps one tile (the long-lead one) in half
    // b = 2 s mod 5 and the other in half b + 1 (mod 5); stage s + 1 sits in
    // halves b + 2 and b + 3, and half b + 4 (stage s - 1's second tile) is
    // free while stage s is consumed. So the long-lead tile of stage s + 2
    // streams into half b + 4 about two stages before it is read, and the
    // other into half b as soon as stage s is consumed, one stage ahead. (Two
    // full 64 KB slots, the most the LDS holds, would give both only one
    // stage.) The activation tile leads for the store and residual
    // projections, the weight tile for the SwiGLU projection (each measured
    // about 1% ahead of the other choice on the block's shapes).
    constexpr bool kALong = EPI != H3_EPI_SWIGLU;
    constexpr int kLongOp = kALong ? 1 : 0;  // dma operand index: 0 W, 1 A
    // LDS byte address of this wave's first slab of half 0.
    const uint32_t lds_wave = lds_addr(smem) + (uint32_t)(8 * wave * 64 * 16);
    // Direct load of slab 8 wave + i of stage kt's W (op 0) or A (op 1) tile
    // into half h.
    auto dma = [&](int h, int op, int i, int kt) {
        const int slab = 8 * wave + i;
        i32x4_t r = op ? rs_a : ((EPI == H3_EPI_SWIGLU && ((slab >> 1) & 1)) ? rs_w2 : rs_w);
        if (kt >= k1) r = rs_none;
        const uint32_t m0 = lds_wave + (uint32_t)((h * kTileChunks + 64 * i) * 16);
        dma_slab(r, m0, op ? a_voff[i] : w_voff[i], kt * BK * 2);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int r32 = lane & 31, g2 = lane >> 5;
    // This wave's MFMA operands of one 16-wide k-step: 4 W and 4 A sub-tiles.
    struct Ops {
        bf16x8_t a[4], w[4];
    };
    // LDS read number r (0..7) of k-step ks of the stage whose W and A tiles
    // are in halves hw and ha, in the order the MFMAs consume the operands:
    // W[0], A[0..3], W[1..3].
    auto read = [&](int hw, int ha, int ks, int r, Ops &o) {
        if (r >= 1 && r <= 4)
            o.a[r - 1] = __builtin_bit_cast(
                bf16x8_t, smem[ha * kTileChunks + swz(wm * 128 + (r - 1) * 32 + r32, ks * 2 + g2)]);
        else {
            const int i = r == 0 ? 0 : r - 4;
            o.w[i] = __builtin_bit_cast(bf16x8_t, smem[hw * kTileChunks + swz(wn * 128 + i * 32 + r32, ks * 2 + g2)]);
        }
    };
    // One k-step (16 MFMAs) of stage kt, whose ring base is b (compile time)
    // and whose operands `cur` already holds. Per k-step:
    //  ks 0..2: read k-step ks+1 of stage kt into `nxt`;
    //  ks 0, 1: also issue the long-lead tile of stage kt+2 into half b+4
    //           (4 loads each, every fourth slot);
    //  ks 3:    wait for stage kt+1 (only the 8 loads of stage kt+2's
    //           long-lead tile may stay in flight), make sure this wave's
    //           reads of stage kt are done, barrier (stage kt+1 visible,
    //           stage kt's halves free), then read k-step 0 of stage kt+1 and
    //           issue the other tile of stage kt+2 into half b.
    // The loads and reads sit between the MFMAs in a fixed order, so issuing
    // them never leaves the matrix pipe idle. Raw barrier: __syncthreads()'s
    // fences would wait for every outstanding load. Reads of a stage at or
    // past k1 see stale or zero data and are never used.
    auto kstep = [&](int kt, int ks, int b, const Ops &cur, Ops &nxt) {
        // the long-lead tile in half b, the other in b + 1 (stage kt + 1: b + 2, b + 3)
        const int hw = kALong ? (b + 1) % 5 : b, ha = kALong ? b : (b + 1) % 5;
        const int hw1 = kALong ? (b + 3) % 5 : (b + 2) % 5, ha1 = kALong ? (b + 2) % 5 : (b + 3) % 5;
        const int hfree = (b + 4) % 5;
        if (ks == 3) {
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int i = t >> 2, j = t & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.w[i], cur.a[j], acc[i][j], 0, 0, 0);
            if (t & 1) {
                if (ks < 2 && (t & 3) == 1) dma(hfree, kLongOp, 4 * ks + (t >> 2), kt + 2);
                if (ks == 3) dma(b, 1 - kLongOp, t >> 1, kt + 2);
            } else {
                if (ks < 3) read(hw, ha, ks + 1, t >> 1, nxt);
                else read(hw1, ha1, 0, t >> 1, nxt);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage = [&](int kt, int b, Ops &r0, Ops &r1) {
        kstep(kt, 0, b, r0, r1);
        kstep(kt, 1, b, r1, r0);
        kstep(kt, 2, b, r0, r1);
        kstep(kt, 3, b, r1, r0);
    };

    // Prologue: stages k0 (halves 0, 1) and k0+1 (halves 2, 3) in flight;
    // stage k0's first k-step in registers.
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) dma(0, kLongOp, i, k0);
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) dma(1, 1 - kLongOp, i, k0);
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) dma(2, kLongOp, i, k0 + 1);
#pragma unroll
    for (int i = 0; i < kSlabsPerWave; ++i) dma(3, 1 - kLongOp, i, k0 + 1);
    Ops opa, opb;
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) read(kALong ? 1 : 0, kALong ? 0 : 1, 0, r, opa);
    // Five stages per iteration bring the ring base back to 0 (b = 0, 2, 4,
    // 1, 3); the remaining 0..4 stages follow with their own bases.
    int kt = k0;
#pragma unroll 1
    for (; kt + 5 <= k1; kt += 5) {
        stage(kt, 0, opa, opb);
        stage(kt + 1, 2, opa, opb);
        stage(kt + 2, 4, opa, opb);
        stage(kt + 3, 1, opa, opb);
        stage(kt + 4, 3, opa, opb);
    }
    if (kt < k1) stage(kt, 0, opa, opb);
    if (kt + 1 < k1) stage(kt + 1, 2, opa, opb);
    if (kt + 2 < k1) stage(kt + 2, 4, opa, opb);
    if (kt + 3 < k1) stage(kt + 3, 1, opa, opb);
    // Drain the loads still in flight (stages past the range) before the
    // workgroup can end or reuse the LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (!PARTIAL && EPI == H3_EPI_SWIGLU) {
        gemm_epilogue<EPI>(p, acc, tm, tn, wm, wn, r32, g2);
    } else if constexpr (!PARTIAL) {
        __syncthreads();  // every wave is done with the ring before it holds the epilogue's tiles
        gemm_epilogue_lds<EPI>(p, acc, tm, tn, wm, wn, lane, smem + wave * kTileChunks);
    } else {
        // FP32 partial sums, register-major: float4 q of thread t at
        // part[(q * 256 + t) * 4], q = (4 i + j) * 4 + e / 4.
        float4 *dst = reinterpret_cast<float4 *>(part);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; e += 4)
                    dst[((4 * i + j) * 4 + e / 4) * kThreads + t] =
                        make_float4(acc[i][j][e], acc[i][j][e + 1], acc[i][j][e + 2], acc[i][j][e + 3]);
    }
}

// The tile (a workgroup index of the XCD-contiguous order) a drawing
// workgroup on XCD `xcd` takes, -1 when none is left: the XCD's own counter
// first (ticket i is tile 8 i + xcd, after the static tickets), then, once
// that is used up, what is left of the other XCDs' (their counters read at
// once, then one with tiles left drawn from). Thread 0 draws; the result
// reaches the other waves through the first word of the LDS ring, between
// barriers.
__device__ __forceinline__ int gemm_draw(const GemmArgs &p, int xcd, uint4 *smem) {
    if (threadIdx.x == 0) {
        const int n = p.dp_tiles, s0 = p.static_tickets;
        int tile = 8 * (s0 + atomicAdd(p.queue + xcd, 1)) + xcd;
        if (tile >= n) {
            int c[8];
#pragma unroll
            for (int y = 0; y < 8; ++y)
                c[y] = __hip_atomic_load(p.queue + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            tile = -1;
#pragma unroll
            for (int d = 1; d < 8; ++d) {
                const int y = (xcd + d) & 7;
                if (tile >= 0 || 8 * (s0 + c[y]) + y >= n) continue;
                const int u = 8 * (s0 + atomicAdd(p.queue + y, 1)) + y;
                if (u < n) tile = u;
            }
        }
        reinterpret_cast<int *>(smem)[0] = tile;
    }
    __syncthreads();
    const int tile = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int *>(smem)[0]);
    __syncthreads();  // every wave has read it before the ring is loaded
    return tile;
}

// Data-parallel tiles: the first dp_tiles tiles of the grouped order,
// XCD-contiguous (workgroups are dealt round-robin over the 8 XCDs, so
// workgroup b is the (b / 8)-th of XCD b % 8 and takes tile b). In long
// launches the last tiles of each XCD's range are drawn instead, by more
// workgroups than tiles: an XCD that runs ahead (XCDs differ by a few percent
// in speed under load) then takes over the end of slower XCDs' ranges
// instead of idling, and the surplus workgroups find nothing and leave.
template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs p) {
    // LDS: the ring of five 32 KB operand tiles (160 KB).
    __shared__ uint4 smem[5 * kTileChunks];
    int bid = blockIdx.x;
    if ((int)(blockIdx.x >> 3) >= p.static_tickets) {
        bid = gemm_draw(p, blockIdx.x & 7, smem);
        if (bid < 0) return;
    }
    int tm, tn;
    gemm_tile_coords(bid, p.tiles_m, p.tiles_n, p.group_m, p.dp_tiles, tm, tn);
    gemm_tile<EPI, false>(p, smem, tm, tn, 0, (int)(p.K / BK), nullptr);
}

// Stream-K tail: workgroup w takes the units [w U / G, (w + 1) U / G) of the
// tail's U = sk_tiles * (K / 64) (tile, stage) units, G = sk_groups; a range
// is shorter than a tile, so it touches at most two tiles, and leaves FP32
// partial sums for each in its two slots of `part`.
template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_sk_kernel(GemmArgs p) {
    __shared__ uint4 smem[5 * kTileChunks];
    const int KT = (int)(p.K / BK);
    const int w = blockIdx.x;
    const int64_t U = (int64_t)p.sk_tiles * KT;
    const int u0 = (int)(w * U / p.sk_groups), u1 = (int)((w + 1) * U / p.sk_groups);
    const int t0 = u0 / KT, t1 = (u1 - 1) / KT;
#pragma unroll 1
    for (int tile = t0; tile <= t1; ++tile) {
        int tm, tn;
        gemm_grouped_coords(p.dp_tiles + tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        const int k0 = tile == t0 ? u0 - tile * KT : 0;
        const int k1 = tile == t1 ? u1 - tile * KT : KT;
        if (tile > t0) __syncthreads();  // every wave is done with the LDS slots
        gemm_tile<EPI, true>(p, smem, tm, tn, k0, k1, p.part + ((int64_t)w * 2 + (tile - t0)) * (BM * BN));
    }
}


// Stream-K fix-up: one wavefront per (tail tile, 128 x 128 quarter, 32-row
// block j of the quarter) sums, in K order, the partial sums of the
// workgroups whose unit ranges cover the tile, then applies the epilogue to
// those rows exactly as the main kernel's wave would. A wave reads 16 float4
// per partial slot, so the pass has many loads in flight across 16 waves per
// tile.
template <int EPI, int J>
__device__ __forceinline__ void gemm_fixup_rows(const GemmArgs &p, int tile, int wave, int lane) {
    const int t = wave * 64 + lane;           // the main kernel's thread
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, g2 = lane >> 5;
    const int KT = (int)(p.K / BK);
    const int64_t U = (int64_t)p.sk_tiles * KT, G = p.sk_groups;
    const int64_t tb = (int64_t)tile * KT, te = tb + KT;
    // workgroup w covers units [w U / G, (w + 1) U / G)
    int64_t w = (tb * G) / U;
    while (w > 0 && (w * U) / G > tb) --w;
    while (((w + 1) * U) / G <= tb) ++w;
    f32x16_t acc[4][4];  // only the column J is used
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][J][e] = 0.f;
    for (; w < G && (w * U) / G < te; ++w) {
        const int64_t ws = (w * U) / G;
        const int sg = ws / KT == tile ? 0 : 1;  // this tile is the workgroup's first or second segment
        const float4 *src = reinterpret_cast<const float4 *>(p.part + (w * 2 + sg) * (BM * BN));
        float4 v[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[i][q] = src[((4 * i + J) * 4 + q) * kThreads + t];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[i][J][4 * q] += v[i][q].x;
                acc[i][J][4 * q + 1] += v[i][q].y;
                acc[i][J][4 * q + 2] += v[i][q].z;
                acc[i][J][4 * q + 3] += v[i][q].w;
            }
    }
    int tm, tn;
    gemm_grouped_coords(p.dp_tiles + tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    gemm_epilogue_rows<EPI, J>(p, acc, tm, tn, wm, wn, r32, g2);
}

template <int EPI>
__global__ __launch_bounds__(64) void gemm_fixup_kernel(GemmArgs p) {
    const int lane = threadIdx.x;
    const int wave = (blockIdx.x >> 2) & 3;   // the quarter: the main kernel's wave
    const int tile = blockIdx.x >> 4;
    switch (blockIdx.x & 3) {                 // 32-row block of the quarter
        case 0: gemm_fixup_rows<EPI, 0>(p, tile, wave, lane); break;
        case 1: gemm_fixup_rows<EPI, 1>(p, tile, wave, lane); break;
        case 2: gemm_fixup_rows<EPI, 2>(p, tile, wave, lane); break;
        default: gemm_fixup_rows<EPI, 3>(p, tile, wave, lane); break;
    }
}

}  // namespace

void launch_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                   uint16_t *c, int64_t ldc, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                   const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
                   int32_t n_mod_groups, const int32_t *mod_idx, hipStream_t stream, void *workspace) {
    if (M_valid <= 0) return;
    GemmArgs p;
    p.a = a; p.w = w; p.bias = bias; p.c = c; p.resid = resid; p.gate = gate; p.mod_idx = mod_idx;
    p.lda = lda; p.ldw = ldw; p.ldc = ldc; p.ld_r = ld_r;
    p.ld_gate = n_mod_groups > 1 ? ld_gate_group : 0;
    p.M = M_valid; p.N = N; p.K = K;
    p.n_groups = n_mod_groups > 0 ? n_mod_groups : 1;
    p.ffn = (int32_t)(N / 2);
    const GemmPlan plan = gemm_plan(M_valid, N, K, epilogue);
    p.tiles_m = plan.tiles_m;
    p.tiles_n = plan.tiles_n;
    // Tile rows per group, measured on the block's projections: wide grids
    // (the SwiGLU FFN) keep the L2 best with 8; narrow ones with 2 at 58,816
    // rows (230 tile rows), 4 at 5,424 (22) and 8 at 4,096 (16).
    p.group_m = (p.tiles_n >= 128 || p.tiles_m <= 16) ? 8 : p.tiles_m <= 32 ? 4 : 2;
    const bool sk = workspace != nullptr && plan.sk_groups > 0;
    p.dp_tiles = sk ? plan.dp_tiles : plan.tiles;
    p.sk_tiles = sk ? plan.sk_tiles : 0;
    p.sk_groups = sk ? plan.sk_groups : 0;
    p.part = static_cast<float *>(workspace);
    p.queue = nullptr;
    p.static_tickets = (p.dp_tiles + 7) / 8;
    dim3 grid((unsigned)p.dp_tiles);
    if (workspace != nullptr && plan.deal) {
        p.queue = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + plan.queue_off);
        p.static_tickets = plan.static_tickets;
        grid = dim3((unsigned)plan.grid);
        launch_zero_rows(reinterpret_cast<uint16_t *>(p.queue), 128, 128, 0, 1, stream);  // the 8 counters
    }
    if (p.dp_tiles > 0) {
        switch (epilogue) {
            case H3_EPI_RESIDUAL: gemm_bf16_kernel<H3_EPI_RESIDUAL><<<grid, kThreads, 0, stream>>>(p); break;
            case H3_EPI_SWIGLU: gemm_bf16_kernel<H3_EPI_SWIGLU><<<grid, kThreads, 0, stream>>>(p); break;
            default: gemm_bf16_kernel<H3_EPI_STORE><<<grid, kThreads, 0, stream>>>(p); break;
        }
    }
    if (!sk) return;
    const dim3 sgrid((unsigned)p.sk_groups);
    switch (epilogue) {
        case H3_EPI_RESIDUAL: gemm_bf16_sk_kernel<H3_EPI_RESIDUAL><<<sgrid, kThreads, 0, stream>>>(p); break;
        case H3_EPI_SWIGLU: gemm_bf16_sk_kernel<H3_EPI_SWIGLU><<<sgrid, kThreads, 0, stream>>>(p); break;
        default: gemm_bf16_sk_kernel<H3_EPI_STORE><<<sgrid, kThreads, 0, stream>>>(p); break;
    }
    const dim3 fgrid((unsigned)p.sk_tiles * 16);
    switch (epilogue) {
        case H3_EPI_RESIDUAL: gemm_fixup_kernel<H3_EPI_RESIDUAL><<<fgrid, 64, 0, stream>>>(p); break;
        case H3_EPI_SWIGLU: gemm_fixup_kernel<H3_EPI_SWIGLU><<<fgrid, 64, 0, stream>>>(p); break;
        default: gemm_fixup_kernel<H3_EPI_STORE><<<fgrid, 64, 0, stream>>>(p); break;
    }
}

}  // namespace h3

using namespace h3;

extern "C" int h3_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                         uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                         int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                         int64_t ld_gate_group, int32_t n_mod_groups, const int32_t *mod_idx, void *workspace,
                         size_t ws_bytes, void *stream) {
    int s = h3_check_linear(a, lda, w, ldw, bias, c, ldc, M_buf, M_valid, N, K, epilogue, resid, ld_r, gate,
                            ld_gate_group, n_mod_groups, workspace, ws_bytes);
    if (s != H3_OK || M_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    launch_linear(a, lda, w, ldw, bias, c, ldc, M_valid, N, K, epilogue, resid, ld_r, gate, ld_gate_group,
                  n_mod_groups, mod_idx, st, workspace);
    launch_zero_rows(c, ldc, epilogue == H3_EPI_SWIGLU ? N / 2 : N, M_valid, M_buf, st);
    return launch_status();
}
