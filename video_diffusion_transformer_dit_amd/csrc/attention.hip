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
//  * V is first staged transposed per head (V^T[head][d][key], keys padded to
//    a multiple of 64) by a small pre-pass, once per distinct K/V segment.
//  * K and V^T stream through LDS in tiles of 64 keys, double-buffered, with
//    gfx950's direct global->LDS buffer loads (16 bytes per lane straight into
//    LDS): no staging registers, and the next tile is in flight while the
//    current one is consumed.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    a lane then holds 16 keys of one query per 32x32 block, which is exactly
//    the B-operand layout the O^T = V^T P^T product needs, so P goes from the
//    score accumulators to the next MFMA without an LDS round trip.
//  * In V^T the keys of every 16-key group are permuted (bits 2 and 3 of the
//    key index swapped) so each lane's 8 keys of a P.V k-step are one 16-byte
//    LDS read.
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
    const uint16_t *sk[H3_MAX_SEGMENTS];   // segment row 0, head 0
    const uint16_t *svt[H3_MAX_SEGMENTS];  // segment's V^T planes [heads][128][lpad]
    int64_t sldk[H3_MAX_SEGMENTS], slpad[H3_MAX_SEGMENTS], slen[H3_MAX_SEGMENTS];
};

// Segment fields held in scalar registers while the segment is streamed.
struct SegState {
    const uint16_t *k, *vt;
    int64_t ldk, lpad, len;
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
    SegState r{a.sk[0], a.svt[0], a.sldk[0], a.slpad[0], a.slen[0]};
#pragma unroll
    for (int j = 1; j < H3_MAX_SEGMENTS; ++j)
        if (j == s) r = SegState{a.sk[j], a.svt[j], a.sldk[j], a.slpad[j], a.slen[j]};
    return r;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Direct global -> LDS load of one 1 KB slab: lane i's 16 bytes (descriptor
// rsrc, byte offset voff + soff) land at slab + 16 i.
__device__ __forceinline__ void load_slab(__amdgpu_buffer_rsrc_t rsrc, const uint4 *slab, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)slab, 16, voff, soff, 0, 0);
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
    // Register-class hints (empty asm, no instruction): the Q operands live in
    // AGPRs, which the MFMA reads directly, leaving VGPRs for scores and P.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+a"(qop[j][ks]));

    f32x16_t oacc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[i][j][e] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(oacc[i][j]));  // O lives in AGPRs
    float l_run[2] = {0.f, 0.f};

    // ---- K / V^T tile loader (direct to LDS). A tile is 16 slabs of K (4 keys
    //      x 16 chunks) and 16 slabs of V^T (8 channels x 8 chunks); wave w
    //      loads slabs 4w .. 4w+3 of each. Lane i of K slab s holds key
    //      4s + i/16, physical chunk i%16 = logical chunk c ^ (key & 15); lane i
    //      of V^T slab s holds channel 8s + i/8, physical chunk i%8. ----
    int k_voff[4], vt_voff[4];
    const int kkey0 = lane >> 4, kp = lane & 15;
    const int vd0 = lane >> 3, vp = lane & 7;

    int n_tiles = 0;
#pragma unroll
    for (int s = 0; s < H3_MAX_SEGMENTS; ++s)
        if (s < a.n_seg) n_tiles += (int)((a.slen[s] + BKV - 1) / BKV);

    // Position of the next tile to load: segment `seg`, key offset `seg_k0`.
    int seg = 0;
    int64_t seg_k0 = 0;
    SegState nS = seg_of(a, 0);
    auto set_offsets = [&](const SegState &S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * (4 * wave + i) + kkey0;
            k_voff[i] = (int)((key * S.ldk + 8 * (kp ^ (key & 15))) * 2);
            const int d = 8 * (4 * wave + i) + vd0;
            vt_voff[i] = (int)((d * S.lpad + 8 * (vp ^ ((d ^ (d >> 3)) & 7))) * 2);
        }
    };
    set_offsets(nS);
    auto load_tile = [&](const SegState &S, int64_t k0, int buf) {
        const int64_t rows = min<int64_t>(S.len - k0, BKV);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(S.k + k0 * S.ldk + head * D, ((rows - 1) * S.ldk + D) * 2);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(S.vt + (int64_t)head * D * S.lpad + k0, (D * S.lpad - k0) * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            load_slab(rk, &k_lds[buf][64 * (4 * wave + i)], k_voff[i], 0);
            load_slab(rv, &v_lds[buf][64 * (4 * wave + i)], vt_voff[i], 0);
        }
    };
    auto advance = [&]() {
        seg_k0 += BKV;
        if (seg_k0 >= nS.len) {
            ++seg;
            seg_k0 = 0;
            if (seg < a.n_seg) {
                nS = seg_of(a, seg);
                set_offsets(nS);
            }
        }
    };

    load_tile(nS, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    int64_t cur_len = nS.len;  // length of the segment the current tile is in
    int64_t cur_k0 = 0;
    advance();

    // Softmax with a per-row reference maximum m_ref (exp2 domain): p =
    // exp2(s c - m_ref) stays <= 2^kSlack while no score exceeds m_ref + kSlack,
    // so the hot loop never rescales O. A tile whose maximum would break that
    // bound makes the wave leave the inner loop before any P.V of the tile,
    // rescale O and l to the new maximum and redo the tile (always at the
    // first tile, rarely afterwards). The redone tile re-issues the same
    // prefetch (identical bytes) and reaches the same barriers, so every wave
    // still passes the same number of barriers.
    constexpr float kSlack = 10.0f;
    float m_ref[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
    int it = 0;
#pragma unroll 1
    while (true) {
        bool brk = false;
        float tmax[2];
#pragma unroll 1
        for (; it < n_tiles; ++it) {
            const int buf = it & 1;
            const bool has_next = it + 1 < n_tiles;
            const int64_t nk0 = seg_k0;
            const int64_t nlen = nS.len;
            if (has_next) load_tile(nS, nk0, buf ^ 1);

            auto qk = [&](int hb, f32x16_t (&sacc)[2]) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) sacc[j][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8_t kop =
                        __builtin_bit_cast(bf16x8_t, k_lds[buf][k_pos(32 * hb + l32, 2 * ks + h)]);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[j][ks], sacc[j], 0, 0, 0);
                }
            };
            auto mask = [&](int hb, f32x16_t (&sacc)[2]) {
                if (cur_k0 + 32 * hb + 32 > cur_len) {  // keys past the segment end
                    const int valid = (int)(cur_len - cur_k0) - 32 * hb;
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int key = 8 * (v >> 2) + 4 * h + (v & 3);
                            if (key >= valid) sacc[j][v] = -__builtin_huge_valf();
                        }
                }
            };
            auto rowmax = [&](const f32x16_t (&sacc)[2], float (&mx)[2]) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float m = sacc[j][0];
#pragma unroll
                    for (int v = 1; v < 16; ++v) m = fmaxf(m, sacc[j][v]);
                    mx[j] = m;
                }
            };
            // P = exp2(s c - m_ref) packed to BF16; row sums returned in `sums`
            // (committed to l only once the tile is known not to be redone).
            auto expo = [&](const f32x16_t (&sacc)[2], bf16x8_t (&pop)[2][2], float (&sums)[2]) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float p[16];
                    float sum = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][v], a.scale_log2, -m_ref[j]));
                        sum += p[v];
                    }
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        uint4 u;
                        u.x = pack_bf16x2(p[8 * s2 + 0], p[8 * s2 + 1]);
                        u.y = pack_bf16x2(p[8 * s2 + 2], p[8 * s2 + 3]);
                        u.z = pack_bf16x2(p[8 * s2 + 4], p[8 * s2 + 5]);
                        u.w = pack_bf16x2(p[8 * s2 + 6], p[8 * s2 + 7]);
                        pop[j][s2] = __builtin_bit_cast(bf16x8_t, u);
                    }
                    sums[j] = sum;
                }
            };
            auto pv = [&](int hb, const bf16x8_t (&pop)[2][2]) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8_t vop =
                            __builtin_bit_cast(bf16x8_t, v_lds[buf][vt_pos(32 * dt + l32, 2 * (2 * hb + s2) + h)]);
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            oacc[dt][j] =
                                __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[j][s2], oacc[dt][j], 0, 0, 0);
                    }
                }
            };
            // Interleave each MFMA with a few VALU instructions of the other
            // half's softmax and the LDS operand read it needs.
#define H3_INTERLEAVE(VALU)                                           \
    do {                                                              \
        _Pragma("unroll") for (int i_ = 0; i_ < 16; ++i_) {           \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        \
            __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);     \
        }                                                             \
    } while (0)

            f32x16_t s0[2], s1[2];
            bf16x8_t p0[2][2], p1[2][2];
            float mx0[2], mx1[2], sum0[2], sum1[2];
            qk(0, s0);                                   // A: S0
            mask(0, s0);
            {                                            // B: S1 || max(S0), P0
                qk(1, s1);
                rowmax(s0, mx0);
                expo(s0, p0, sum0);
                H3_INTERLEAVE(8);
            }
            mask(1, s1);
            rowmax(s1, mx1);
            bool over = false;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float m = fmaxf(mx0[j], mx1[j]);
                m = fmaxf(m, __shfl_xor(m, 32)) * a.scale_log2;
                tmax[j] = m;
                over |= m > m_ref[j] + kSlack;
            }
            if (__any(over)) {  // leave before any P.V of this tile
                brk = true;
                break;
            }
            {                                            // C: O += V0 P0 || P1
                pv(0, p0);
                expo(s1, p1, sum1);
                H3_INTERLEAVE(7);
            }
            pv(1, p1);                                   // D: O += V1 P1
#pragma unroll
            for (int j = 0; j < 2; ++j) l_run[j] += sum0[j] + sum1[j];

            if (has_next) {
                cur_len = nlen;
                cur_k0 = nk0;
                advance();
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's slabs landed
            __syncthreads();                                   // all slabs visible, buf free
        }
        if (!brk) break;
        // Rare path: raise the reference maximum and rescale O and l.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float m_new = fmaxf(m_ref[j], tmax[j]);
            const float alpha = __builtin_amdgcn_exp2f(m_ref[j] - m_new);
            m_ref[j] = m_new;
            l_run[j] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][j][e] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(oacc[dt][j]));
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

// V -> V^T staging for one segment: tile of 64 keys x 128 channels of one head
// through LDS; output rows are channels, keys permuted inside 16-key groups
// (kperm) and zero-filled past the segment end.
__global__ __launch_bounds__(256) void vt_transpose_kernel(const uint16_t *v, int64_t ld_v, int64_t len,
                                                           uint16_t *vt, int64_t lpad) {
    __shared__ uint16_t tile[BKV][D + 8];  // +8: row stride 272 B
    const int64_t k0 = (int64_t)blockIdx.x * BKV;
    const int head = blockIdx.y;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = t + 256 * j;
        const int key = idx >> 4, c = idx & 15;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (k0 + key < len) val = *reinterpret_cast<const uint4 *>(v + (k0 + key) * ld_v + head * D + 8 * c);
        *reinterpret_cast<uint4 *>(&tile[key][8 * c]) = val;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = t + 256 * j;
        const int d = idx >> 3, c = idx & 7;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = tile[kperm(8 * c + i)][d];
        uint4 out;
        out.x = e[0] | ((uint32_t)e[1] << 16);
        out.y = e[2] | ((uint32_t)e[3] << 16);
        out.z = e[4] | ((uint32_t)e[5] << 16);
        out.w = e[6] | ((uint32_t)e[7] << 16);
        *reinterpret_cast<uint4 *>(vt + ((int64_t)head * D + d) * lpad + k0 + 8 * c) = out;
    }
}

}  // namespace

void launch_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                      int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len, int32_t heads,
                      float softmax_scale, const h3_qgroup *groups, int32_t n_groups, void *workspace,
                      hipStream_t stream) {
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    // The dense case is one group over [0, valid_len) attending to keys [0, valid_len).
    h3_qgroup dense = {};
    const bool is_dense = groups == nullptr;
    if (is_dense) {
        dense.q_begin = 0;
        dense.q_end = valid_len;
        dense.n_seg = 1;
        dense.seg[0] = h3_kv_seg{nullptr, nullptr, 0, 0, valid_len};
        groups = &dense;
        n_groups = valid_len > 0 ? 1 : 0;
    }
    // Stage V^T once per distinct segment.
    VtPlan plan;
    vt_plan(is_dense ? nullptr : groups, is_dense ? 0 : n_groups, valid_len, heads, &plan);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    for (int i = 0; i < plan.n; ++i) {
        const VtSeg &e = plan.seg[i];
        const uint16_t *src = e.own ? v + e.begin * ld_v : e.v + e.begin * e.ld;
        const int64_t ld = e.own ? ld_v : e.ld;
        vt_transpose_kernel<<<dim3((unsigned)(e.lpad / BKV), (unsigned)heads), 256, 0, stream>>>(
            src, ld, e.len, reinterpret_cast<uint16_t *>(ws + e.off), e.lpad);
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
            const VtSeg &e = plan.seg[plan.map[gi][s]];
            if (ss.k == nullptr) {
                a.sk[s] = k + ss.begin * ld_k;
                a.sldk[s] = ld_k;
            } else {
                a.sk[s] = ss.k + ss.begin * ss.ld;
                a.sldk[s] = ss.ld;
            }
            a.svt[s] = reinterpret_cast<const uint16_t *>(ws + e.off);
            a.slpad[s] = e.lpad;
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
                            int32_t n_groups, void *workspace, size_t ws_bytes, void *stream) {
    int s = h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim,
                               softmax_scale, groups, n_groups, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, softmax_scale, groups, n_groups,
                     workspace, (hipStream_t)stream);
    return launch_status();
}
