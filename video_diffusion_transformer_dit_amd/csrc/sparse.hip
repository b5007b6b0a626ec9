// Sol-Attn block selection for gfx950 (Sol-H3 report, §3.4 "Sparse
// Attention").
//
// What it computes: the sequence is [prefix | target] with the prefix rows
// [0, P). Target queries are cut into blocks of 256 rows and target keys into
// blocks of 64 rows, both counted from P (the last block of each may be
// short). For each head and query block b, every target KV block j gets the
// score s_bj = mean_q(b) . mean_k(j) / sqrt(128). The blocks with
// s_bj > mu_b + tau * sigma_b are selected, where mu_b and sigma_b are the
// mean and the population standard deviation of s_b. over j. The output is,
// per (head, b), the ascending list of selected j and its length. The
// attention kernel's list mode consumes these lists.
//
// How:
//  * sparse_pool_kernel: the mean of each block's q rows and of each KV
//    block's k rows, in FP32. A workgroup owns one block and 2048 columns
//    (16 heads). Each thread sums 8 columns over the block's rows with
//    coalesced 128-bit loads, so q and k are read once. Query means are
//    stored [head][block][128]. KV means are stored transposed,
//    [head][128][n_kb_pad], so the selection reads them coalesced.
//  * sparse_select_kernel: a workgroup owns 8 query blocks of one head, with
//    their means in LDS. Thread t scores the contiguous KV blocks
//    [t m, t m + m), m = n_kb_pad / 256, with float4 loads of the transposed
//    means. Scores stay in registers. Two block-wide reductions give mu and
//    sigma, and a block-wide exclusive scan of the per-thread counts places
//    each thread's selected indices, so every list comes out ascending.
#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int D = 128;
constexpr int kPoolCols = 2048;   // columns per pooling workgroup (256 threads x 8)
constexpr int kQg = 8;            // query blocks per selection workgroup
constexpr int kMaxPer = 16;       // KV blocks per selection thread (H3_SPARSE_MAX_KBLOCKS / 256)

struct PoolArgs {
    const uint16_t *q, *k;
    int64_t ld_q, ld_k;
    int64_t P, T;        // prefix rows, target rows
    int32_t cols;        // heads * 128
    int32_t n_qb, n_kb, n_kb_pad;
    float *qbar;         // [heads][n_qb][128]
    float *kbarT;        // [heads][128][n_kb_pad]
};

__global__ __launch_bounds__(256) void sparse_pool_kernel(PoolArgs a) {
    const int x = blockIdx.x;
    const bool is_q = x < a.n_qb;
    const int blk = is_q ? x : x - a.n_qb;
    const int bs = is_q ? H3_SPARSE_Q_BLOCK : H3_SPARSE_K_BLOCK;
    const int64_t r0 = (int64_t)blk * bs;
    const int n = (int)min<int64_t>(bs, a.T - r0);
    const int col = blockIdx.y * kPoolCols + 8 * threadIdx.x;
    if (col >= a.cols) return;
    const uint16_t *src = is_q ? a.q : a.k;
    const int64_t ld = is_q ? a.ld_q : a.ld_k;
    const uint16_t *p = src + (a.P + r0) * ld + col;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int r = 0;
    for (; r + 4 <= n; r += 4) {
        uint4 u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)(r + i) * ld);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float f[8];
            unpack8(u[i], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += f[e];
        }
    }
    for (; r < n; ++r) {
        float f[8];
        unpack8(*reinterpret_cast<const uint4 *>(p + (int64_t)r * ld), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f[e];
    }
    const float fn = (float)n;
    const int head = col / D, c = col % D;
    if (is_q) {
        float *dst = a.qbar + ((int64_t)head * a.n_qb + blk) * D + c;
        *reinterpret_cast<float4 *>(dst) = make_float4(acc[0] / fn, acc[1] / fn, acc[2] / fn, acc[3] / fn);
        *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4] / fn, acc[5] / fn, acc[6] / fn, acc[7] / fn);
    } else {
        float *dst = a.kbarT + ((int64_t)head * D + c) * a.n_kb_pad + blk;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[(int64_t)e * a.n_kb_pad] = acc[e] / fn;
    }
}

struct SelArgs {
    const float *qbar, *kbarT;
    int32_t n_qb, n_kb, n_kb_pad, per;  // per = n_kb_pad / 256 (multiple of 4, <= kMaxPer)
    float tau, scale;
    uint16_t *blocks;    // [heads][n_qb][n_kb]
    int32_t *counts;     // [heads][n_qb]
};

// Sum over the 256 threads of kQg values at once; every thread gets the totals.
__device__ __forceinline__ void block_sum8(float (&v)[kQg], float (*red)[kQg]) {
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
#pragma unroll
    for (int g = 0; g < kQg; ++g) v[g] = wave_sum(v[g]);
    if (lane == 0)
#pragma unroll
        for (int g = 0; g < kQg; ++g) red[w][g] = v[g];
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kQg; ++g) v[g] = (red[0][g] + red[1][g]) + (red[2][g] + red[3][g]);
    __syncthreads();
}

__global__ __launch_bounds__(256) void sparse_select_kernel(SelArgs a) {
    __shared__ float qs[kQg][D];
    __shared__ float red[4][kQg];
    __shared__ int wsum[4][kQg];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int head = blockIdx.y;
    const int b0 = blockIdx.x * kQg;
    const int nb = min(kQg, a.n_qb - b0);
    for (int i = t; i < kQg * D; i += 256) {
        const int g = i / D, c = i % D;
        qs[g][c] = g < nb ? a.qbar[((int64_t)head * a.n_qb + b0 + g) * D + c] : 0.f;
    }
    __syncthreads();

    // scores of this thread's KV blocks j = j0 .. j0 + per - 1
    const int j0 = t * a.per;
    float sc[kMaxPer][kQg];
    const float *kt = a.kbarT + (int64_t)head * D * a.n_kb_pad + j0;
#pragma unroll
    for (int i4 = 0; i4 < kMaxPer / 4; ++i4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int g = 0; g < kQg; ++g) sc[4 * i4 + e][g] = 0.f;
        if (4 * i4 < a.per) {
            for (int c = 0; c < D; ++c) {
                const float4 kv = *reinterpret_cast<const float4 *>(kt + (int64_t)c * a.n_kb_pad + 4 * i4);
#pragma unroll
                for (int g = 0; g < kQg; ++g) {
                    const float qv = qs[g][c];
                    sc[4 * i4 + 0][g] = __builtin_fmaf(qv, kv.x, sc[4 * i4 + 0][g]);
                    sc[4 * i4 + 1][g] = __builtin_fmaf(qv, kv.y, sc[4 * i4 + 1][g]);
                    sc[4 * i4 + 2][g] = __builtin_fmaf(qv, kv.z, sc[4 * i4 + 2][g]);
                    sc[4 * i4 + 3][g] = __builtin_fmaf(qv, kv.w, sc[4 * i4 + 3][g]);
                }
            }
        }
    }
    // mean and population standard deviation over the n_kb valid blocks
    const float fn = (float)a.n_kb;
    float mu[kQg], sd[kQg];
#pragma unroll
    for (int g = 0; g < kQg; ++g) mu[g] = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i)
#pragma unroll
        for (int g = 0; g < kQg; ++g) {
            sc[i][g] *= a.scale;
            if (i < a.per && j0 + i < a.n_kb) mu[g] += sc[i][g];
        }
    block_sum8(mu, red);
#pragma unroll
    for (int g = 0; g < kQg; ++g) {
        mu[g] /= fn;
        sd[g] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i)
#pragma unroll
        for (int g = 0; g < kQg; ++g) {
            const float d = sc[i][g] - mu[g];
            if (i < a.per && j0 + i < a.n_kb) sd[g] = __builtin_fmaf(d, d, sd[g]);
        }
    block_sum8(sd, red);
    float thr[kQg];
#pragma unroll
    for (int g = 0; g < kQg; ++g) thr[g] = mu[g] + a.tau * sqrtf(sd[g] / fn);

    // selection: per-thread counts, block-wide exclusive scan, ascending write
    int cnt[kQg];
#pragma unroll
    for (int g = 0; g < kQg; ++g) {
        cnt[g] = 0;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < a.per && j0 + i < a.n_kb && sc[i][g] > thr[g]) ++cnt[g];
    }
    int incl[kQg];
#pragma unroll
    for (int g = 0; g < kQg; ++g) {
        int v = cnt[g];
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int u = __shfl_up(v, m);
            if (lane >= m) v += u;
        }
        incl[g] = v;
        if (lane == 63) wsum[w][g] = v;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < kQg; ++g) {
        if (g >= nb) continue;
        int base = 0;
        for (int ww = 0; ww < w; ++ww) base += wsum[ww][g];
        int off = base + incl[g] - cnt[g];
        uint16_t *row = a.blocks + ((int64_t)head * a.n_qb + b0 + g) * a.n_kb;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i)
            if (i < a.per && j0 + i < a.n_kb && sc[i][g] > thr[g]) row[off++] = (uint16_t)(j0 + i);
        if (t == 255) a.counts[(int64_t)head * a.n_qb + b0 + g] = base + incl[g];
    }
}

}  // namespace

void launch_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, int64_t valid_len,
                          int64_t prefix_len, int32_t heads, float tau, uint16_t *blocks, int32_t *counts,
                          void *workspace, hipStream_t stream) {
    SparseGeom g;
    sparse_geometry(valid_len, prefix_len, heads, &g);
    if (g.T == 0) return;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    PoolArgs pa;
    pa.q = q;
    pa.k = k;
    pa.ld_q = ld_q;
    pa.ld_k = ld_k;
    pa.P = prefix_len;
    pa.T = g.T;
    pa.cols = heads * D;
    pa.n_qb = (int32_t)g.n_qb;
    pa.n_kb = (int32_t)g.n_kb;
    pa.n_kb_pad = (int32_t)g.n_kb_pad;
    pa.qbar = reinterpret_cast<float *>(ws + g.qbar_off);
    pa.kbarT = reinterpret_cast<float *>(ws + g.kbar_off);
    sparse_pool_kernel<<<dim3((unsigned)(g.n_qb + g.n_kb), (unsigned)((pa.cols + kPoolCols - 1) / kPoolCols)), 256,
                         0, stream>>>(pa);
    SelArgs sa;
    sa.qbar = pa.qbar;
    sa.kbarT = pa.kbarT;
    sa.n_qb = pa.n_qb;
    sa.n_kb = pa.n_kb;
    sa.n_kb_pad = pa.n_kb_pad;
    sa.per = (int32_t)g.per;
    sa.tau = tau;
    sa.scale = 1.0f / sqrtf((float)D);
    sa.blocks = blocks;
    sa.counts = counts;
    sparse_select_kernel<<<dim3((unsigned)((g.n_qb + kQg - 1) / kQg), (unsigned)heads), 256, 0, stream>>>(sa);
}

}  // namespace h3

using namespace h3;

extern "C" size_t h3_sparse_select_workspace_bytes(int64_t valid_len, int64_t prefix_len, int32_t heads) {
    if (valid_len < 0 || prefix_len < 0 || prefix_len > valid_len || heads <= 0) return 0;
    SparseGeom g;
    sparse_geometry(valid_len, prefix_len, heads, &g);
    return g.T == 0 ? 0 : g.ws_bytes;
}

extern "C" int h3_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                                int64_t valid_len, int64_t prefix_len, int32_t heads, int32_t head_dim, float tau,
                                uint16_t *blocks, int32_t *counts, void *workspace, size_t ws_bytes,
                                void *stream) {
    int s = h3_check_sparse_select(q, ld_q, k, ld_k, valid_len, prefix_len, heads, head_dim, tau, blocks, counts,
                                   workspace, ws_bytes);
    if (s != H3_OK || valid_len == prefix_len) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_sparse_select(q, ld_q, k, ld_k, valid_len, prefix_len, heads, tau, blocks, counts, workspace,
                         (hipStream_t)stream);
    return launch_status();
}
