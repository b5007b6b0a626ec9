// Exact multi-head attention over a long packed sequence for gfx950.
//
// What it computes: per head, o = softmax(q k^T * scale) v over the keys of
// the query's group (Sol-H3 report, §3.2: dense SDPA attention over the packed
// QKV in the flat (total, heads, head_dim) layout; vLLM-Omni H3 blog, §3.1:
// the backend receives the valid length and drops the padding suffix;
// SolarWM H3 Realtime, stages 2-3: condition/audio/video query groups, video
// queries reading a pre-concatenated history K/V plus the current chunk).
//
// How (flash-style, one pass, the L^2 score matrix never exists):
//  * A workgroup of 4 wavefronts owns 256 queries of one head; each wavefront
//    owns 64 queries, kept in registers as MFMA operands.
//  * K and V stream through LDS in tiles of 64 keys, double-buffered: the next
//    tile's global loads are in flight while the current one is consumed.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of one query per 32x32 block, which is exactly
//    the B-operand layout the O^T = V^T P^T product needs, so P goes from the
//    score accumulators to the next MFMA without an LDS round trip.
//  * V is stored transposed in LDS (V^T[d][key]) with the keys of every
//    16-key group permuted (bits 2 and 3 of the key index swapped) so each
//    lane's 8 keys of a P.V k-step are one 16-byte read.
//  * Online softmax in FP32 in the exp2 domain (scale * log2 e folded into one
//    FMA); the O accumulator is rescaled only when some row maximum grew.
//    P is rounded to BF16 for the P.V MFMA.
//  * Workgroups are dealt round-robin over the 8 XCDs; work items are remapped
//    so each XCD walks a contiguous range (consecutive query tiles of one
//    head), so the workgroups resident on an XCD stream the same K/V through
//    its L2.
#include <algorithm>
#include <utility>

#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

constexpr int D = 128;          // head dim
constexpr int BQ = 256;         // queries per workgroup
constexpr int WQ = 64;          // queries per wavefront
constexpr int BKV = 64;         // keys per tile
constexpr int kThreads = 256;

// One launch per query group: rows [0, rows) of q/o (already offset to the
// group's first row) attend over n_seg K/V segments in order.
struct AttnArgs {
    const uint16_t *q;
    uint16_t *o;
    int64_t ld_q, ld_o;
    int64_t rows;
    int32_t heads;
    int32_t tiles_per_head;  // ceil(rows / BQ)
    int32_t n_seg;
    float scale_log2;        // softmax scale * log2(e)
    const uint16_t *sk[H3_MAX_SEGMENTS];  // segment row 0, head 0
    const uint16_t *sv[H3_MAX_SEGMENTS];
    int64_t sldk[H3_MAX_SEGMENTS], sldv[H3_MAX_SEGMENTS], slen[H3_MAX_SEGMENTS];
};

// Segment fields held in scalar registers while the segment is streamed.
struct SegState {
    const uint16_t *k, *v;
    int64_t ldk, ldv, len;
};

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

// LDS layouts (16-byte chunks):
//  K tile  [64 keys][16 chunks]: chunk c of key r at c ^ (r & 15).
//  V^T tile [128 d][8 chunks]  : logical chunk c of row d at c ^ ((d ^ (d >> 3)) & 7);
//                                keys inside a 16-key group permuted by kperm.
__device__ __forceinline__ int k_pos(int key, int c) { return key * 16 + (c ^ (key & 15)); }
__device__ __forceinline__ int vt_pos(int d, int c) { return d * 8 + (c ^ ((d ^ (d >> 3)) & 7)); }
__device__ __forceinline__ int kperm(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Fields of segment s, read from the kernel arguments at static offsets
// under a uniform condition (dynamic indexing would go through memory).
__device__ __forceinline__ SegState seg_of(const AttnArgs &a, int s) {
    SegState r{a.sk[0], a.sv[0], a.sldk[0], a.sldv[0], a.slen[0]};
#pragma unroll
    for (int j = 1; j < H3_MAX_SEGMENTS; ++j)
        if (j == s) r = SegState{a.sk[j], a.sv[j], a.sldk[j], a.sldv[j], a.slen[j]};
    return r;
}

__device__ __forceinline__ uint32_t perm_lo(uint32_t x, uint32_t y) {  // lo16(x) | lo16(y) << 16
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t x, uint32_t y) {  // hi16(x) | hi16(y) << 16
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__global__ __launch_bounds__(kThreads, 1) void attention_fwd_kernel(AttnArgs a) {
    __shared__ uint4 k_lds[2][BKV * 16];  // 2 x 16 KB
    __shared__ uint4 v_lds[2][D * 8];     // 2 x 16 KB

    // ---- work item: (head, group, query tile) with XCD-contiguous order ----
    const int total = a.tiles_per_head * a.heads;
    int bid = blockIdx.x;
    {
        const int q8 = total / 8, rr = total % 8;
        const int xcd = bid % 8, local = bid / 8;
        bid = xcd < rr ? xcd * (q8 + 1) + local : rr * (q8 + 1) + (xcd - rr) * q8 + local;
    }
    const int head = bid / a.tiles_per_head;
    const int tile = bid - head * a.tiles_per_head;
    const int64_t q0 = (int64_t)tile * BQ;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t qw = q0 + wave * WQ;  // this wave's first query

    // ---- Q operands: Qop[j][ks] = Q[qw + 32j + l32][8(2ks + h) .. +7] ----
    bf16x8_t qop[2][8];
    {
        const int64_t rows = a.rows - qw;  // may be <= 0 for idle waves
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(a.q + qw * a.ld_q + head * D, rows > 0 ? ((min<int64_t>(rows, WQ) - 1) * a.ld_q + D) * 2 : 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                qop[j][ks] = __builtin_bit_cast(
                    bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                  rq, (int)(((32 * j + l32) * a.ld_q + 8 * (2 * ks + h)) * 2), 0, 0));
    }

    f32x16_t oacc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[i][j][e] = 0.f;
    float m_run[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
    float l_run[2] = {0.f, 0.f};

    // ---- K/V tile loader: thread t loads K rows (t>>4) + 16 i, chunk t & 15,
    //      and V rows 4 (t>>4) + i, chunk t & 15 (i < 4) ----
    const int ld_r = t >> 4, ld_c = t & 15;
    uint4 kst[4], vst[4];

    // Count tiles over all segments.
    int n_tiles = 0;
#pragma unroll
    for (int s = 0; s < H3_MAX_SEGMENTS; ++s)
        if (s < a.n_seg) n_tiles += (int)((a.slen[s] + BKV - 1) / BKV);

    // Position of the next tile to load: segment `seg`, key offset `seg_k0`.
    int seg = 0;
    int64_t seg_k0 = 0;
    SegState nS = seg_of(a, 0);
    auto load_tile = [&](const SegState &S, int64_t k0) {
        const int64_t rows = min<int64_t>(S.len - k0, BKV);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(S.k + k0 * S.ldk + head * D, ((rows - 1) * S.ldk + D) * 2);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(S.v + k0 * S.ldv + head * D, ((rows - 1) * S.ldv + D) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kst[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(((ld_r + 16 * i) * S.ldk + 8 * ld_c) * 2), 0, 0));
            vst[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(((4 * ld_r + i) * S.ldv + 8 * ld_c) * 2), 0, 0));
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) k_lds[buf][k_pos(ld_r + 16 * i, ld_c)] = kst[i];
        // V^T: for channel d = 8 ld_c + e, keys 4 ld_r .. +3 (permuted position)
        const int kp = kperm(4 * ld_r);
        uint2 *vt = reinterpret_cast<uint2 *>(&v_lds[buf][0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * ld_c + e;
            const int w = e >> 1;
            const uint32_t x0 = (&vst[0].x)[w], x1 = (&vst[1].x)[w], x2 = (&vst[2].x)[w], x3 = (&vst[3].x)[w];
            uint2 pk;
            if (e & 1) {
                pk.x = perm_hi(x0, x1);
                pk.y = perm_hi(x2, x3);
            } else {
                pk.x = perm_lo(x0, x1);
                pk.y = perm_lo(x2, x3);
            }
            // 8-byte slot: chunk kp / 8, half (kp % 8) / 4
            vt[2 * vt_pos(d, kp >> 3) + ((kp & 7) >> 2)] = pk;
        }
    };
    auto advance = [&]() {
        seg_k0 += BKV;
        if (seg_k0 >= nS.len) {
            ++seg;
            seg_k0 = 0;
            if (seg < a.n_seg) nS = seg_of(a, seg);
        }
    };

    load_tile(nS, 0);
    store_tile(0);
    __syncthreads();

    int64_t cur_len = nS.len;  // length of the segment the current tile is in
    int64_t cur_k0 = 0;
    advance();
#pragma unroll 1
    for (int it = 0; it < n_tiles; ++it) {
        const int buf = it & 1;
        const bool has_next = it + 1 < n_tiles;
        const int64_t nk0 = seg_k0;
        const int64_t nlen = nS.len;
        if (has_next) load_tile(nS, nk0);
        __builtin_amdgcn_sched_barrier(0);

        // ---- S^T = K Q^T: sacc[i][j] keys 32i.., queries 32j.. ----
        f32x16_t sacc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[i][j][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, k_lds[buf][k_pos(32 * i + l32, 2 * ks + h)]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    sacc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[j][ks], sacc[i][j], 0, 0, 0);
            }
        }

        // ---- mask keys past the segment end (last tile of a segment only) ----
        if (cur_k0 + BKV > cur_len) {
            const int valid = (int)(cur_len - cur_k0);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                        if (key >= valid) sacc[i][j][v] = -__builtin_huge_valf();
                    }
        }

        // ---- online softmax (exp2 domain) ----
        bf16x8_t pop[2][4];  // P^T operands: [query tile j][key step s]
        bool need_rescale = false;
        float alpha[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float mx = sacc[0][j][0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[0][j][v]);
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[1][j][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[j], mx * a.scale_log2);
            alpha[j] = __builtin_amdgcn_exp2f(m_run[j] - m_new);
            need_rescale |= m_new > m_run[j];
            m_run[j] = m_new;
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float p[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i][j][v], a.scale_log2, -m_new));
                    sum += p[v];
                }
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    uint4 u;
                    u.x = pack_bf16x2(p[8 * sh + 0], p[8 * sh + 1]);
                    u.y = pack_bf16x2(p[8 * sh + 2], p[8 * sh + 3]);
                    u.z = pack_bf16x2(p[8 * sh + 4], p[8 * sh + 5]);
                    u.w = pack_bf16x2(p[8 * sh + 6], p[8 * sh + 7]);
                    pop[j][2 * i + sh] = __builtin_bit_cast(bf16x8_t, u);
                }
            }
            l_run[j] = l_run[j] * alpha[j] + sum;
        }
        if (__any(need_rescale)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[dt][j][e] *= alpha[j];
        }

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, v_lds[buf][vt_pos(32 * dt + l32, 2 * s + h)]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    oacc[dt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[j][s], oacc[dt][j], 0, 0, 0);
            }
        }

        if (has_next) {
            store_tile(buf ^ 1);
            cur_len = nlen;
            cur_k0 = nk0;
            advance();
        }
        __syncthreads();
    }

    // ---- normalise and store: lane holds O[q][32 dt + 8 g + 4 h + (0..3)] ----
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
        const float inv = 1.0f / l_tot;
        const int64_t q = qw + 32 * j + l32;
        if (q < a.rows) {
            uint16_t *orow = a.o + q * a.ld_o + head * D;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * dt + 8 * g + 4 * h;
                    *reinterpret_cast<uint2 *>(orow + d) =
                        make_uint2(pack_bf16x2(oacc[dt][j][4 * g] * inv, oacc[dt][j][4 * g + 1] * inv),
                                   pack_bf16x2(oacc[dt][j][4 * g + 2] * inv, oacc[dt][j][4 * g + 3] * inv));
                }
        }
    }
}

}  // namespace

void launch_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                      int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len, int32_t heads,
                      float softmax_scale, const h3_qgroup *groups, int32_t n_groups, hipStream_t stream) {
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    // The dense case is one group over [0, valid_len) attending to keys [0, valid_len).
    h3_qgroup dense = {};
    if (groups == nullptr) {
        dense.q_begin = 0;
        dense.q_end = valid_len;
        dense.n_seg = 1;
        dense.seg[0] = h3_kv_seg{nullptr, nullptr, 0, 0, valid_len};
        groups = &dense;
        n_groups = valid_len > 0 ? 1 : 0;
    }
    std::pair<int64_t, int64_t> cov[H3_MAX_GROUPS];
    int nc = 0;
    for (int gi = 0; gi < n_groups; ++gi) {
        const h3_qgroup &g = groups[gi];
        if (g.q_end <= g.q_begin) continue;
        cov[nc++] = {g.q_begin, g.q_end};
        AttnArgs a = {};
        a.q = q + g.q_begin * ld_q;
        a.o = o + g.q_begin * ld_o;
        a.ld_q = ld_q;
        a.ld_o = ld_o;
        a.rows = g.q_end - g.q_begin;
        a.heads = heads;
        a.tiles_per_head = (int32_t)((a.rows + BQ - 1) / BQ);
        a.n_seg = g.n_seg;
        a.scale_log2 = scale * 1.4426950408889634f;
        for (int s = 0; s < g.n_seg; ++s) {
            const h3_kv_seg &ss = g.seg[s];
            if (ss.k == nullptr) {
                a.sk[s] = k + ss.begin * ld_k;
                a.sv[s] = v + ss.begin * ld_v;
                a.sldk[s] = ld_k;
                a.sldv[s] = ld_v;
            } else {
                a.sk[s] = ss.k + ss.begin * ss.ld;
                a.sv[s] = ss.v + ss.begin * ss.ld;
                a.sldk[s] = ss.ld;
                a.sldv[s] = ss.ld;
            }
            a.slen[s] = ss.len;
        }
        attention_fwd_kernel<<<dim3((unsigned)(a.tiles_per_head * heads)), kThreads, 0, stream>>>(a);
    }
    // Zero the rows of o outside every group (the padding suffix included).
    std::sort(cov, cov + nc);
    int64_t prev = 0;
    for (int i = 0; i < nc; ++i) {
        launch_zero_rows(o, ld_o, (int64_t)heads * D, prev, cov[i].first, stream);
        prev = cov[i].second;
    }
    launch_zero_rows(o, ld_o, (int64_t)heads * D, prev, L_buf, stream);
}

}  // namespace h3

using namespace h3;

extern "C" int h3_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                            int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len,
                            int32_t heads, int32_t head_dim, float softmax_scale, const h3_qgroup *groups,
                            int32_t n_groups, void *stream) {
    int s = h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim,
                               softmax_scale, groups, n_groups);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, softmax_scale, groups, n_groups,
                     (hipStream_t)stream);
    return launch_status();
}
