// The attention kernel template for gfx950 and the launch arguments its
// host code fills in. Included by attention.hip (host code and the
// online-softmax instances) and by attention_fixed.hip (the fixed-reference
// instances, built with MFMAs that accumulate the scores in VGPRs).
//
// H3_ATTN_SCORES_IN_VGPR (0 or 1, set by the including source before this
// header) chooses the register class of the score accumulators: 1 keeps
// them in VGPRs, where the softmax reads them without a copy out of the
// accumulator registers, and needs the source to be built with the VGPR MFMA
// form; 0 keeps them in AGPRs next to Q and O.
#pragma once

#include <algorithm>

#include "h3_device.h"
#include "h3_runtime.h"

#ifndef H3_ATTN_SCORES_IN_VGPR
#error "define H3_ATTN_SCORES_IN_VGPR (0 or 1) before including h3_attention_kernel.h"
#endif

namespace h3 {


constexpr int D = 128;          // head dim
constexpr int BQ = 256;         // queries per workgroup
constexpr int WQ = 64;          // queries per wavefront
constexpr int BKV = 64;         // keys per tile
constexpr int kThreads = 256;

// A query group: rows [0, rows) of q/o (offset to the group's first row)
// attend over n_seg K/V segments in order.
struct AttnGroup {
    const uint16_t *q;
    uint16_t *o;
    int64_t rows;
    int32_t tiles_per_head;  // ceil(rows / BQ)
    int32_t n_seg;
    const uint16_t *sk[H3_MAX_SEGMENTS];   // segment row 0, head 0
    const uint16_t *svt[H3_MAX_SEGMENTS];  // segment's V^T planes [heads][128][lpad]
    int64_t sldk[H3_MAX_SEGMENTS], slpad[H3_MAX_SEGMENTS], slen[H3_MAX_SEGMENTS];
};

// One launch covers every query group of a call, as ranges of work items
// (the host's attention schedule): range i owns the items [end[i-1], end[i])
// and covers count[i] (head, tile) items of group grp[group[i]] from item
// first[i] on, each cut into split[i] pieces by key range. Pieces write
// unnormalised partial results (O in FP32 and the row's reference m and sum
// l) to `part`, which the merge pass combines. The longest items run first,
// so short groups and pieces fill the tail instead of running as launches of
// their own.
struct AttnArgs {
    int64_t ld_q, ld_o;
    int32_t heads;
    float scale_log2;        // softmax scale * log2(e)
    int32_t n_ranges;
    int32_t rng_end[H3_MAX_GROUPS + 1], rng_group[H3_MAX_GROUPS + 1], rng_first[H3_MAX_GROUPS + 1],
        rng_count[H3_MAX_GROUPS + 1], rng_split[H3_MAX_GROUPS + 1];
    float *part;             // [records][256][128] FP32 O, then [records][256] (m, l)
    int32_t part_records;
    AttnGroup grp[H3_MAX_GROUPS];
    const float *kmax2;      // [heads] largest squared key norm over all segments
    int32_t *flags;          // items the fixed-reference instance left to the online one (queue word 8 of them)
    int32_t *queue;          // kAttnQueueWords work-queue words, zero when the fixed-reference instance starts
    int32_t n_items;         // work items of the launch
    int32_t static_tickets;  // per XCD: tickets dealt by workgroup index; later ones are drawn from the counter
    // Block-sparse (list) mode: q and o point at row 0; segment 0 is the
    // prefix [0, P), segment 1 the target rows [P, P + T). Work items
    // [0, pre_items) are prefix query tiles (dense over both segments; items
    // past heads * pre_tiles are idle), the rest target query tiles
    // (tiles_per_head per head), which read segment 1 through their list.
    const uint16_t *blocks;  // [heads][tiles_per_head][n_kb] selected KV blocks
    const int32_t *counts;   // [heads][tiles_per_head]
    int32_t n_kb, pre_tiles, pre_items;
    int64_t prefix_len, tgt_rows;
};

// Work-queue words: [0, 8) the ticket counter of each XCD, then the count of
// items left to the online instance, then the online instance's counter.
constexpr int kQueueDeferred = 8, kQueueOnline = 9;
static_assert(kAttnQueueWords >= 10, "work-queue words");
// Work-item dealing of a launch of n items. Launches of fewer than 8 rounds
// of the chip's slots deal every item by workgroup index (the grid is the n
// items). Longer ones deal all but the last 96 tickets of each XCD (3 rounds
// of its 32 slots) that way and let the rest be drawn from the counters, with
// up to 64 surplus workgroups per XCD: XCDs differ in speed by a few percent
// under load, which over a long launch adds up to more than an item.
struct AttnDeal {
    int grid, static_tickets;
};
inline AttnDeal attn_deal(int n) {
    if (n < 8 * kAttnSlots) return {n, (n + 7) / 8};
    return {n + std::min(512, (n + 7) / 8 * 8), n / 8 - 96};
}


// The fixed-reference instances, built in attention_fixed.hip: one range of
// work items (dense / list mode), and several ranges (query groups, key-range
// pieces).
void launch_attention_fixed(bool sparse, dim3 grid, const AttnArgs &a, hipStream_t stream);
void launch_attention_fixed_multi(dim3 grid, const AttnArgs &a, hipStream_t stream);

namespace {

// Segment fields held in scalar registers while the segment is streamed.
struct SegState {
    const uint16_t *k, *vt;
    int64_t ldk, lpad, len;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    // Wave-uniform by construction; readfirstlane keeps it in scalar registers.
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int32_t n = __builtin_amdgcn_readfirstlane(bytes >= 0xFFFFFFFFll ? (int32_t)0xFFFFFFFF : (int32_t)bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}

// Maximum / sum of a value over the lane pair (l, l ^ 32), in every lane
// (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
__device__ __forceinline__ SegState seg_of(const AttnGroup &a, int s) {
    SegState r{a.sk[0], a.svt[0], a.sldk[0], a.slpad[0], a.slen[0]};
#pragma unroll
    for (int j = 1; j < H3_MAX_SEGMENTS; ++j)
        if (j == s) r = SegState{a.sk[j], a.svt[j], a.sldk[j], a.slpad[j], a.slen[j]};
    return r;
}

// K / V^T tile stream: position (segment, first key) of the next tile to load.
// In list mode, li is the list index of the tile and nxt (a VGPR holding a
// wave-uniform value) the first key of the following list entry, read from
// LDS one tile ahead so that no LDS wait sits on the load path.
struct Cursor {
    int seg;
    int k0, len;  // first key of the tile, keys in the segment (32-bit: scalar compares)
    SegState S;
    int li, nxt;
};

// The work item a workgroup on XCD `xcd` draws (-1: none left); thread 0
// only. The fixed-reference instance draws its own XCD's items first (word
// xcd counts the tickets drawn past the static ones; ticket i is item
// 8 i + xcd), then what is left of the other XCDs' (their counters are read
// at once, then one with items left is drawn from). The online instance
// walks the list of items the fixed one left to it, and reads the counts
// before it draws, so that when nothing was left (the usual case) its
// workgroups leave without an atomic.
template <bool FIXED>
__device__ __forceinline__ int attn_claim(const AttnArgs &a, int xcd) {
    const int n = a.n_items, s0 = a.static_tickets;
    if (FIXED) {
        int item = 8 * (s0 + atomicAdd(a.queue + xcd, 1)) + xcd;
        if (item < n) return item;
        int c[8];
#pragma unroll
        for (int y = 0; y < 8; ++y)
            c[y] = __hip_atomic_load(a.queue + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int d = 1; d < 8; ++d) {
            const int y = (xcd + d) & 7;
            if (8 * (s0 + c[y]) + y >= n) continue;
            item = 8 * (s0 + atomicAdd(a.queue + y, 1)) + y;
            if (item < n) return item;
        }
        return -1;
    }
    const int left = __hip_atomic_load(a.queue + kQueueDeferred, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int drawn = __hip_atomic_load(a.queue + kQueueOnline, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (drawn >= left) return -1;
    const int i = atomicAdd(a.queue + kQueueOnline, 1);
    return i < left ? a.flags[i] : -1;
}

// The dense / grouped kernel (SPARSE = false) and the block-sparse list mode
// (SPARSE = true) share every step; list mode only changes which query tile a
// workgroup owns and which key tiles of segment 1 it visits.
//
// A workgroup takes one work item as it starts. Workgroups are dealt
// round-robin over the 8 XCDs, so workgroup b is the (b / 8)-th of XCD b % 8.
// In the fixed-reference instance, the first static_tickets of each XCD take
// ticket b / 8 (item b) at once; later ones draw theirs. With surplus
// workgroups, an XCD that runs ahead starts its next workgroups sooner and
// takes over the items of slower ones; the surplus finds nothing left and
// leaves. No workgroup waits on another.
template <bool SPARSE, bool FIXED, bool MULTI>
__global__ __launch_bounds__(kThreads, 1) void attention_fwd_kernel(AttnArgs a) {
    int item = blockIdx.x;
    if (!FIXED || (int)(blockIdx.x >> 3) >= a.static_tickets) {
        __shared__ int claimed;
        if (threadIdx.x == 0) claimed = attn_claim<FIXED>(a, blockIdx.x & 7);
        __syncthreads();
        item = __builtin_amdgcn_readfirstlane(claimed);
        if (item < 0) return;
    }
    int ri = 0;  // the item's range (wave-uniform; range 0 unless MULTI)
    if (MULTI)
        while (ri + 1 < a.n_ranges && item >= a.rng_end[ri]) ++ri;
    const AttnGroup &G = a.grp[MULTI ? a.rng_group[ri] : 0];
    constexpr int KB = BKV * 16;  // 16-byte chunks per K tile buffer (16 KB)
    constexpr int VB = D * 8;     // chunks per V^T tile buffer (16 KB)
    // K buffers 0, 1 then V^T buffers 0, 1.
    __shared__ uint4 smem[2 * KB + 2 * VB];
    // List mode: the work item's selected tiles as first keys within segment 1.
    __shared__ int lst[SPARSE ? H3_SPARSE_MAX_KBLOCKS + 1 : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
    const int l32 = lane & 31, h = lane >> 5;

    // ---- work item: (head, query tile) with XCD-contiguous order ----
    int head;
    const uint16_t *qbase;  // the tile's first query row, head 0
    uint16_t *obase;
    int64_t rows_left;      // query rows from qbase to the end of the tile's group
    bool listed = false;    // list mode, target tile: segment 1 through the list
    int lcount = 0;
    int pieces = 1, piece = 0, rec = 0;  // key-range pieces of the item; this one; its partial record
    {
        int bid = item;
        if (SPARSE && bid < a.pre_items) {
            if (bid >= a.heads * a.pre_tiles) return;  // idle item
            head = bid / a.pre_tiles;
            const int64_t q0 = (int64_t)(bid - head * a.pre_tiles) * BQ;
            qbase = G.q + q0 * a.ld_q;
            obase = G.o + q0 * a.ld_o;
            rows_left = a.prefix_len - q0;
        } else {
            const int total = G.tiles_per_head * a.heads;
            if (!MULTI) {
                if (SPARSE) bid -= a.pre_items;  // pre_items is a multiple of 8: same XCD
                const int q8 = total / 8, rr = total % 8;
                const int xcd = bid % 8, local = bid / 8;
                bid = xcd < rr ? xcd * (q8 + 1) + local : rr * (q8 + 1) + (xcd - rr) * q8 + local;
            } else {
                // the range's items start at a multiple of 8 and span a multiple of 8
                const int item0 = ri > 0 ? a.rng_end[ri - 1] : 0;
                const int span = a.rng_end[ri] - item0;
                const int local = bid - item0;
                const int idx = (local % 8) * (span / 8) + local / 8;
                pieces = a.rng_split[ri];
                if (idx >= a.rng_count[ri] * pieces) return;  // padding item
                piece = idx % pieces;
                rec = idx;
                bid = a.rng_first[ri] + idx / pieces;
            }
            head = bid / G.tiles_per_head;
            const int tile = bid - head * G.tiles_per_head;
            const int64_t q0 = (SPARSE ? a.prefix_len : 0) + (int64_t)tile * BQ;
            qbase = G.q + q0 * a.ld_q;
            obase = G.o + q0 * a.ld_o;
            rows_left = (SPARSE ? a.prefix_len + a.tgt_rows : G.rows) - q0;
            if (SPARSE) {
                listed = true;
                const int64_t item = (int64_t)head * G.tiles_per_head + tile;
                lcount = min(max(a.counts[item], 0), a.n_kb);
                const uint16_t *src = a.blocks + item * a.n_kb;
                // Entries past the last block become an empty tile at the
                // segment end (no load, every key masked).
                const int tl = (int)a.tgt_rows;
                for (int i = t; i <= lcount; i += kThreads)
                    lst[i] = i < lcount ? (src[i] < a.n_kb ? BKV * (int)src[i] : tl) : tl;
                __syncthreads();
            }
        }
    }
    const int64_t qw = wave * WQ;  // this wave's first query, relative to qbase

    // ---- Q operands: qop[j][ks] = Q[qw + 32j + l32][8(2ks + h) .. +7] ----
    bf16x8_t qop[2][8];
    {
        const int64_t rows = rows_left - qw;  // may be <= 0 for idle waves
        const __amdgpu_buffer_rsrc_t rqb =
            make_rsrc(qbase + qw * a.ld_q + head * D, rows > 0 ? ((min<int64_t>(rows, WQ) - 1) * a.ld_q + D) * 2 : 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                qop[j][ks] = __builtin_bit_cast(
                    bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                  rqb, (int)(((32 * j + l32) * a.ld_q + 8 * (2 * ks + h)) * 2), 0, 0));
    }
    // Score bound per query row (exp2 domain): B = |q| max|k| scale log2(e),
    // with a 2^-10 margin for the FP32 rounding of the norms. The lane pair
    // (l, l ^ 32) holds the two halves of a row. With B <= 30 and the
    // reference taken from the first half tile, p stays in [2^-60, 2^60].
    constexpr float kFixedMax = 30.0f;
    float bound[2];
    {
        const float km = a.kmax2[head];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float s2 = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const uint4 u = __builtin_bit_cast(uint4, qop[j][ks]);
                float f[8];
                unpack8(u, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) s2 = __builtin_fmaf(f[e], f[e], s2);
            }
            bound[j] = sqrtf(pair_sum(s2) * km) * a.scale_log2 * (1.0f + 1.0f / 1024.0f);
        }
    }
    if (FIXED) {
        // the workgroup takes the fixed reference only if all its rows allow it
        __shared__ int vote[4];
        const int ok = __all(bound[0] <= kFixedMax && bound[1] <= kFixedMax);
        if (lane == 0) vote[wave] = ok;
        __syncthreads();
        const bool wg_ok = vote[0] && vote[1] && vote[2] && vote[3];
        if (!wg_ok) {  // left to the online instance
            if (t == 0) a.flags[atomicAdd(a.queue + kQueueDeferred, 1)] = item;
            return;
        }
    }
    // Register-class hints (empty asm, no instruction): Q and O live in AGPRs,
    // which the MFMA reads directly, leaving the VGPRs for scores and P.
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
        for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(oacc[i][j]));
    // Row sums of p as two running partial sums per query block (even and
    // odd keys of each pair), added together at the end.
    float sa[2] = {0.f, 0.f}, sb[2] = {0.f, 0.f};

    // ---- tile loads (direct to LDS). A K tile is 16 slabs of 4 keys x 16
    //      chunks, a V^T tile 16 slabs of 8 channels x 8 chunks; wave w loads
    //      slabs 4w .. 4w+3 of each. Lane i of K slab s holds key 4s + i/16,
    //      physical chunk i%16 = logical chunk c ^ (key & 15); lane i of V^T
    //      slab s holds channel 8s + i/8, physical chunk i%8. ----
    const int kkey0 = lane >> 4, kp = lane & 15;
    const int vd0 = lane >> 3, vp = lane & 7;
    const uint32_t lds0 = lds_addr(smem);
    int n_tiles = 0;
#pragma unroll
    for (int s = 0; s < H3_MAX_SEGMENTS; ++s)
        if (s < G.n_seg && !(listed && s == 1)) n_tiles += (int)((G.slen[s] + BKV - 1) / BKV);
    if (listed) n_tiles += lcount;
    // A piece covers key tiles [kt0, kt1) of the group's key sequence.
    int seg0 = 0, t0 = 0;
    if (MULTI && pieces > 1) {
        const int kt0 = piece * n_tiles / pieces;
        n_tiles = (piece + 1) * n_tiles / pieces - kt0;
        t0 = kt0;
#pragma unroll
        for (int s = 0; s < H3_MAX_SEGMENTS; ++s) {
            const int ts = (int)((G.slen[s] + BKV - 1) / BKV);
            if (seg0 == s && s + 1 < G.n_seg && t0 >= ts) {
                t0 -= ts;
                seg0 = s + 1;
            }
        }
    }

    // Two cursors over the same tile sequence: K runs two tiles ahead of the
    // tile being finished, V^T one tile ahead.
    const SegState S0 = seg_of(G, seg0);
    Cursor kc{seg0, BKV * t0, (int)S0.len, S0, 0, 0}, vc{seg0, BKV * t0, (int)S0.len, S0, 0, 0};
    int k_voff[4], v_voff[4];
    auto set_k = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * (4 * wave + i) + kkey0;
            k_voff[i] = (int)((key * kc.S.ldk + 8 * (kp ^ (key & 15))) * 2);
        }
    };
    auto set_v = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 8 * (4 * wave + i) + vd0;
            v_voff[i] = (int)((d * vc.S.lpad + 8 * (vp ^ ((d ^ (d >> 3)) & 7))) * 2);
        }
    };
    set_k();
    set_v();
    auto advance = [&](Cursor &c, bool is_k) {
        if (SPARSE && listed && c.seg == 1) {  // next list entry (prefetched)
            if (++c.li < lcount) {
                c.k0 = __builtin_amdgcn_readfirstlane(c.nxt);
                c.nxt = lst[c.li + 1 <= lcount ? c.li + 1 : lcount];
            } else {
                c.seg = G.n_seg;
            }
            return;
        }
        c.k0 += BKV;
        if (c.k0 >= c.len) {
            ++c.seg;
            c.k0 = 0;
            if (c.seg < G.n_seg) {
                c.S = seg_of(G, c.seg);
                c.len = (int)c.S.len;
                if (is_k) set_k();
                else set_v();
                if (SPARSE && listed) {  // entering segment 1: first list entry
                    c.li = 0;
                    if (lcount > 0) {
                        c.k0 = __builtin_amdgcn_readfirstlane(lst[0]);
                        c.nxt = lst[1];
                    } else {
                        c.seg = G.n_seg;
                    }
                }
            }
        }
    };
    // Keys of the cursor's tile that exist (64 past the last tile: nothing to mask).
    auto valid_keys = [&](const Cursor &c) -> int {
        return c.seg < G.n_seg ? min(c.len - c.k0, BKV) : BKV;
    };
    // Issue this wave's 4 slab loads of the cursor's tile into buffer b. Past
    // the last tile the descriptor has length zero: the loads return zero and
    // touch no memory, so every iteration issues the same loads.
    auto issue_k = [&](int b, int half) {
        const int rows = min(kc.len - kc.k0, BKV);
        i32x4_t r = raw_rsrc(kc.S.k + (int64_t)kc.k0 * kc.S.ldk + head * D, ((int64_t)(rows - 1) * kc.S.ldk + D) * 2);
        if (kc.seg >= G.n_seg || rows <= 0) r.z = 0;
#pragma unroll
        for (int i = 2 * half; i < 2 * half + 2; ++i)
            dma_slab(r, lds0 + (uint32_t)((b * KB + 64 * (4 * wave + i)) * 16), k_voff[i], 0);
    };
    auto issue_v = [&](int b, int half) {
        i32x4_t r = raw_rsrc(vc.S.vt + (int64_t)head * D * vc.S.lpad + vc.k0, ((int64_t)D * vc.S.lpad - vc.k0) * 2);
        if (vc.seg >= G.n_seg) r.z = 0;
#pragma unroll
        for (int i = 2 * half; i < 2 * half + 2; ++i)
            dma_slab(r, lds0 + (uint32_t)((2 * KB + b * VB + 64 * (4 * wave + i)) * 16), v_voff[i], 0);
    };

    // ---- per-lane LDS read offsets (bytes); buffer and sub-tile offsets are
    //      instruction immediates ----
    // K operand of k-step ks: key l32 (+32 per half), logical chunk 2 ks + h.
    int koff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) koff[ks] = (k_pos(l32, 2 * ks + h)) * 16;
    // V^T operand: channel 32 dt + l32, logical chunk 2 (2 hb + s2) + h; the
    // swizzle depends on dt only through its parity.
    int voff[2][4];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) voff[par][c4] = (2 * KB + vt_pos(32 * par + l32, 2 * c4 + h)) * 16;
    const char *lds_bytes = reinterpret_cast<const char *>(smem);
    // K operand number pr = 16 hb' ... : half hb = pr / 8, k-step ks = pr % 8.
    auto kop_read = [&](int b, int pr) -> bf16x8_t {
        const int hb = pr >> 3, ks = pr & 7;
        return __builtin_bit_cast(bf16x8_t,
                                  *reinterpret_cast<const uint4 *>(lds_bytes + koff[ks] + (b * KB + hb * 512) * 16));
    };
    // V^T operand number pr: half hb = pr / 8, 16-key group s2 = (pr / 4) % 2,
    // channel block dt = pr % 4.
    auto vop_read = [&](int b, int pr) -> bf16x8_t {
        const int hb = pr >> 3, s2 = (pr >> 2) & 1, dt = pr & 3;
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                lds_bytes + voff[dt & 1][2 * hb + s2] + (b * VB + (dt >> 1) * 512) * 16));
    };

    // The key loop runs over half tiles u (32 keys: tile u/2, half u%2).
    // Scores S^T of a half tile, [query block j]: lane holds query 32 j + l32,
    // keys 8 (v/4) + 4 h + v%4 of the half. The MFMAs accumulate them in sacc
    // (AGPRs, or VGPRs with H3_ATTN_SCORES_IN_VGPR); the softmax works on a
    // shifted copy (sv).
    f32x16_t sacc[2], sv[2];
    auto pin_sacc = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#if H3_ATTN_SCORES_IN_VGPR
            asm volatile("" : "+v"(sacc[j]));
#else
            asm volatile("" : "+a"(sacc[j]));
#endif
        }
    };
    // Scores of keys >= valid (within the half) -> -inf; `in_acc`: the
    // accumulators themselves, one 16-register block at a time.
    auto mask = [&](f32x16_t (&s)[2], int valid, bool in_acc) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = 8 * (v >> 2) + 4 * h + (v & 3);
                if (key >= valid) s[j][v] = -__builtin_huge_valf();
            }
            if (in_acc) {  // keep the block in the accumulators' register class
#if H3_ATTN_SCORES_IN_VGPR
                asm volatile("" : "+v"(s[j]));
#else
                asm volatile("" : "+a"(s[j]));
#endif
            }
        }
    };
    // Per-lane maximum of a half tile's raw scores, per query block.
    float tmaxr[2];

    // ---- prologue: K of tiles 0 and 1, V^T of tile 0; S of half 0 ----
    issue_k(0, 0);
    issue_k(0, 1);
    advance(kc, true);
    issue_k(1, 0);
    issue_k(1, 1);
    advance(kc, true);
    issue_v(0, 0);
    issue_v(0, 1);
    int vk_cur = valid_keys(vc);  // valid keys of the current tile
    int vk_next = BKV;            // ... of the next one (set when its V^T is issued)
    advance(vc, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kop = kop_read(0, ks);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[j][ks], ks == 0 ? f32x16_t{} : sacc[j], 0, 0,
                                                              0);
    }
    pin_sacc();
#pragma unroll
    for (int j = 0; j < 2; ++j) sv[j] = sacc[j];
    if (vk_cur < 32) mask(sv, vk_cur, false);

    // Softmax with a per-row reference maximum m_ref (exp2 domain). The
    // scores are kept shifted, y = s c - m_ref, so p = exp2(y). m_ref starts
    // at the first half tile's maximum (half 0 always has a valid key), in
    // both forms. In the online form, while no y exceeds kSlack, p <= 2^kSlack
    // and O and l need no rescaling; a half tile whose maximum y breaks the
    // bound raises m_ref and rescales O, l and its own y before any of its P
    // is formed, so nothing is ever recomputed. In the fixed form the score
    // bound already keeps every y in [-60, 60]. The slack only has to keep O
    // finite: O <= 2^kSlack * keys * max|v|, which at 2^31 keys still leaves
    // |v| up to 2^57; the wider it is, the rarer the wave-wide rescales (with
    // 10, scores of standard deviation 11.5 in the exp2 domain rescaled often
    // enough to cost 4% at 58,758 keys and 20% at 4,096).
    constexpr float kSlack = 40.0f;
    float m_ref[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        {
            float m = sv[j][0];
#pragma unroll
            for (int v = 1; v < 16; ++v) m = fmaxf(m, sv[j][v]);
            m_ref[j] = pair_max(m) * a.scale_log2;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) sv[j][v] = __builtin_fmaf(sv[j][v], a.scale_log2, -m_ref[j]);
        tmaxr[j] = 0.f;
    }

    // One half tile u = 2t + odd (uu = u % 4, so the tile parity tp = uu / 2
    // and the buffers are compile-time): the shifted scores y of half u are
    // in sv, their per-lane maximum in tmaxr.
    //   check  half u's maximum y against kSlack, rescale if needed;
    //   sync   even u: V^T of tile t has landed, every wave is done with V^T of
    //          tile t-1 -> load V^T of tile t+1 into that buffer;
    //          odd u:  K of tile t+1 has landed, every wave is done with K of
    //          tile t -> load K of tile t+2 into that buffer.
    //          The other operand's 4 loads may stay in flight (vmcnt 4).
    //   X      S of half u+1 = K Q^T into sacc (16 MFMAs) || p = exp2(y) in sv
    //          and BF16 P of half u || this half's 4 loads;
    //   mask   keys past the segment end in half u+1 (last tile of a segment);
    //   Y      O += V^T P^T of half u (16 MFMAs) || row sums of half u, then
    //          sv = y of half u+1 and its maximum.
    // Each phase is 16 slots of one MFMA plus its share of the other work, in
    // a fixed order (sched_barrier); the empty asm statements keep each slot's
    // VALU work in its slot. Past the last tile the loads return zero and the
    // scores of half u+1 go unused.
    auto hiter = [&](int uu, bool fixed) {
        const int tp = uu >> 1, odd = uu & 1;
        // check (tmaxr: per-lane maximum of half u's shifted scores); with a
        // fixed reference no score can exceed it
        if (!fixed) {
            bool over = false;
            float tm[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                tm[j] = pair_max(tmaxr[j]);
                over |= tm[j] > kSlack;
            }
            if (__any(over)) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float d = fmaxf(tm[j], 0.f);
                    const float alpha = __builtin_amdgcn_exp2f(-d);
                    m_ref[j] += d;
                    sa[j] *= alpha;
                    sb[j] *= alpha;
#pragma unroll
                    for (int v = 0; v < 16; ++v) sv[j][v] -= d;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[dt][j][e] *= alpha;
                        asm volatile("" : "+a"(oacc[dt][j]));
                    }
                }
            }
        }
        // sync
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        i32x4_t rl;
        int voffs[4];
        uint32_t m0b;
        if (odd) {
            const int rows = min(kc.len - kc.k0, BKV);
            rl = raw_rsrc(kc.S.k + (int64_t)kc.k0 * kc.S.ldk + head * D, ((int64_t)(rows - 1) * kc.S.ldk + D) * 2);
            if (kc.seg >= G.n_seg || rows <= 0) rl.z = 0;
            m0b = lds0 + (uint32_t)((tp * KB + 64 * 4 * wave) * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) voffs[i] = k_voff[i];
        } else {
            rl = raw_rsrc(vc.S.vt + (int64_t)head * D * vc.S.lpad + vc.k0, ((int64_t)D * vc.S.lpad - vc.k0) * 2);
            if (vc.seg >= G.n_seg) rl.z = 0;
            m0b = lds0 + (uint32_t)((2 * KB + (tp ^ 1) * VB + 64 * 4 * wave) * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) voffs[i] = v_voff[i];
            vk_next = valid_keys(vc);
        }

        // X: QK of half u+1 (K buffer of tile (u+1)/2, key half (u+1)%2)
        const int kb = odd ? (tp ^ 1) : tp, khb = odd ? 0 : 1;
        bf16x8_t pop[2][2];  // [j][s2]: keys 16 s2 .. +15 of the half, query block j
        bf16x8_t kop[8];
        // Softmax numerators p = exp2(y) of half u, staggered over the slots
        // so no slot waits on its own results: slot w = 8 gj + e takes exp2
        // of score pair w and the BF16 pack of pair w-1.
        uint32_t pk[16];
        auto pack_pair = [&](int w) {
            const int gj = w >> 3, e = w & 7;
            pk[w] = pack_bf16x2(sv[gj][2 * e], sv[gj][2 * e + 1]);
            asm volatile("" : "+v"(pk[w]));
        };
        kop[0] = kop_read(kb, 8 * khb + 0);
        kop[1] = kop_read(kb, 8 * khb + 1);
        kop[2] = kop_read(kb, 8 * khb + 2);
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) {
            const int ks = sl >> 1, j = sl & 1;
            sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qop[j][ks], ks == 0 ? f32x16_t{} : sacc[j], 0,
                                                              0, 0);
            if (j == 0 && ks + 3 < 8) kop[ks + 3] = kop_read(kb, 8 * khb + ks + 3);
            if ((sl & 3) == 1) dma_slab(rl, m0b + (uint32_t)(64 * 16 * (sl >> 2)), voffs[sl >> 2], 0);
            {
                const int gj = sl >> 3, e = sl & 7;
                sv[gj][2 * e] = __builtin_amdgcn_exp2f(sv[gj][2 * e]);
                sv[gj][2 * e + 1] = __builtin_amdgcn_exp2f(sv[gj][2 * e + 1]);
                asm volatile("" : "+v"(sv[gj][2 * e]), "+v"(sv[gj][2 * e + 1]));
                if (sl >= 1) pack_pair(sl - 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        pack_pair(15);
#pragma unroll
        for (int gj = 0; gj < 2; ++gj)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int w = 8 * gj + 4 * s2;
                pop[gj][s2] = __builtin_bit_cast(bf16x8_t, make_uint4(pk[w], pk[w + 1], pk[w + 2], pk[w + 3]));
            }
        pin_sacc();
        if (odd) {
            advance(kc, true);
        } else {
            advance(vc, false);
        }

        // mask: half u+1 is the second half of tile t (even u) or the first
        // half of tile t+1 (odd u)
        {
            const int valid = odd ? min(vk_next, 32) : vk_cur - 32;
            if (valid < 32) mask(sacc, valid, true);
        }

        // Y: PV of half u (V^T buffer of tile t, key half odd)
        bf16x8_t vop[8];
        vop[0] = vop_read(tp, 8 * odd + 0);
        vop[1] = vop_read(tp, 8 * odd + 1);
        vop[2] = vop_read(tp, 8 * odd + 2);
        // Row sums of half u and the shifted copy / maximum of half u+1,
        // staggered: slot w adds p pair w (two partial sums per query block),
        // stores pair w-1 of the new scores from sacc into sv as y = s c -
        // m_ref (pair w-1 was summed the slot before) and takes the maximum
        // of pair w-2.
        float mx[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
        auto copy_pair = [&](int w) {
            const int gj = w >> 3, e = w & 7;
            sv[gj][2 * e] = __builtin_fmaf(sacc[gj][2 * e], a.scale_log2, -m_ref[gj]);
            sv[gj][2 * e + 1] = __builtin_fmaf(sacc[gj][2 * e + 1], a.scale_log2, -m_ref[gj]);
            asm volatile("" : "+v"(sv[gj][2 * e]), "+v"(sv[gj][2 * e + 1]));
        };
        auto max_pair = [&](int w) {
            const int gj = w >> 3, e = w & 7;
            mx[gj] = fmaxf(mx[gj], fmaxf(sv[gj][2 * e], sv[gj][2 * e + 1]));
            asm volatile("" : "+v"(mx[gj]));
        };
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) {
            const int pr = sl >> 1, j = sl & 1, s2 = pr >> 2, dt = pr & 3;
            oacc[dt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[pr], pop[j][s2], oacc[dt][j], 0, 0, 0);
            if (j == 0 && pr + 3 < 8) vop[pr + 3] = vop_read(tp, 8 * odd + pr + 3);
            {
                const int gj = sl >> 3, e = sl & 7;
                sa[gj] += sv[gj][2 * e];
                sb[gj] += sv[gj][2 * e + 1];
                asm volatile("" : "+v"(sa[gj]), "+v"(sb[gj]));
                if (sl >= 1) copy_pair(sl - 1);
                if (!fixed && sl >= 2) max_pair(sl - 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        copy_pair(15);
        if (!fixed) {
            max_pair(14);
            max_pair(15);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!fixed) tmaxr[j] = mx[j];
        }
        if (odd) vk_cur = vk_next;
    };

    const int n_half = 2 * n_tiles;
    int u = 0;
#pragma unroll 1
    for (; u + 4 <= n_half; u += 4) {
        hiter(0, FIXED);
        hiter(1, FIXED);
        hiter(2, FIXED);
        hiter(3, FIXED);
    }
    if (u < n_half) {
        hiter(0, FIXED);
        hiter(1, FIXED);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // loads past the end

    if (MULTI && pieces > 1) {
        // ---- a piece: unnormalised O rows and (m, l) into its partial record ----
        float *po = a.part + (int64_t)rec * BQ * D;
        float2 *pml = reinterpret_cast<float2 *>(a.part + (int64_t)a.part_records * BQ * D) + (int64_t)rec * BQ;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float l_tot = pair_sum(sa[j] + sb[j]);
            const int r = (int)qw + 32 * j + l32;
            if (r < rows_left) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<float4 *>(po + (int64_t)r * D + 32 * dt + 8 * g + 4 * h) =
                            make_float4(oacc[dt][j][4 * g], oacc[dt][j][4 * g + 1], oacc[dt][j][4 * g + 2],
                                        oacc[dt][j][4 * g + 3]);
                if (h == 0) pml[r] = make_float2(m_ref[j], l_tot);
            }
        }
        return;
    }

    // ---- normalise and store: lane holds O[q][32 dt + 8 g + 4 h + (0..3)].
    //      Launches of several ranges (short items: query groups, key-range
    //      pieces) store through LDS: each wave writes its 64 rows x 128
    //      channels in BF16 to its own 16 KB of the now idle K / V^T buffers
    //      ([64 rows][16 chunks of 8 channels], chunk c of row r at c ^
    //      (r & 15)) and stores them back row by row, 16 bytes per lane, which
    //      shortens a short item's tail (measured -1 to -2% at 4,096 keys
    //      with the scores in AGPRs). The instances with VGPR scores store
    //      directly: there the LDS path pushed part of O into VGPRs, and the
    //      direct form measured 1% faster on the streaming chunk's call; the
    //      one-range dense instance also stores directly (with the scores in
    //      AGPRs the LDS path had cost it 0.5%). ----
    if constexpr (MULTI && !H3_ATTN_SCORES_IN_VGPR) {
        __syncthreads();  // every wave is done with the K / V^T buffers
        uint2 *lo = reinterpret_cast<uint2 *>(smem + wave * (D * 8));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float inv = 1.0f / pair_sum(sa[j] + sb[j]);
            const int row = 32 * j + l32;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int chunk = 4 * dt + g;
                    lo[(row * 16 + (chunk ^ (row & 15))) * 2 + h] =
                        make_uint2(pack_bf16x2(oacc[dt][j][4 * g] * inv, oacc[dt][j][4 * g + 1] * inv),
                                   pack_bf16x2(oacc[dt][j][4 * g + 2] * inv, oacc[dt][j][4 * g + 3] * inv));
                }
        }
        const uint4 *li = smem + wave * (D * 8);
        const int c = lane & 15;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int row = it * 4 + (lane >> 4);
            const int64_t q = qw + row;
            const uint4 val = li[row * 16 + (c ^ (row & 15))];
            if (q < rows_left) *reinterpret_cast<uint4 *>(obase + q * a.ld_o + head * D + 8 * c) = val;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float l_tot = pair_sum(sa[j] + sb[j]);
            const float inv = 1.0f / l_tot;
            const int64_t q = qw + 32 * j + l32;
            if (q < rows_left) {
                uint16_t *orow = obase + q * a.ld_o + head * D;
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
}

}  // namespace
}  // namespace h3
