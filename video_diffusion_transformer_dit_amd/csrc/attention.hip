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
//  * Softmax in FP32 in the exp2 domain (scale * log2 e folded into one FMA),
//    against a per-row reference m: p = exp2(s c - m), with m the row's
//    largest scaled score in the first half tile of keys. By Cauchy-Schwarz
//    every score obeys |s c| <= B = |q| max|k| c, so when B <= 30 every
//    later s c - m lies in [-2B, 2B]: no p leaves [2^-60, 2^60] (normal in
//    FP32 and BF16), and m stays fixed, with no running maximum, check or
//    rescaling. |q| comes from the workgroup's own Q registers, max|k| from
//    the call's keys. The two forms are two instances of the kernel, launched
//    back to back on the same grid: the fixed-reference instance handles
//    every workgroup whose rows all have B <= 30 and flags the others, which
//    the online instance then handles (m starts the same way and is raised,
//    with O rescaled, only when some row maximum grew); it exits at once for
//    the rest. P is rounded to BF16 for the P.V MFMA. The key that sets m
//    gets p within 2^-19 of 1, so BF16(p) = 1: with one valid key both forms
//    return that key's value exactly.
//  * The kernel template is in h3_attention_kernel.h. The fixed-reference
//    instances are built in attention_fixed.hip with the VGPR form of the
//    MFMA instructions, so their score accumulators are VGPRs that the
//    softmax reads in place; the online instances, built here, keep them in
//    AGPRs next to Q and O.
//  * Workgroups are dealt round-robin over the 8 XCDs, and work items are
//    remapped so each XCD walks a contiguous range (consecutive query tiles
//    of one head): the workgroups resident on an XCD stream the same K/V
//    through its L2. In long launches the last rounds of each XCD's range are
//    drawn from a per-XCD ticket counter by more workgroups than items, so an
//    XCD that runs ahead takes over what is left of the others' ranges
//    instead of idling.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <utility>

#define H3_ATTN_SCORES_IN_VGPR 0
#include "h3_attention_kernel.h"

namespace h3 {
namespace {

// Largest squared key norm per head over rows [0, rows) of k, merged into
// kmax2[head] (non-negative FP32 bit patterns compare like unsigned integers,
// so an integer atomic maximum merges them). Workgroup (x, y) owns the rows
// [x per, (x + 1) per) of heads [8 y, 8 y + 8): 128 chunks of 16 bytes per
// row. Thread t takes chunk t & 127 of the rows of parity t >> 7, 8 rows in
// flight; the 16 chunks of one head are 16 consecutive lanes. `per`
// (norm_rows_per_wg) keeps the row blocks at about 128 or fewer, so each
// head's maximum takes at most about 256 atomics.
constexpr int kNormHeads = 8;
int norm_rows_per_wg(int64_t rows) {
    const int64_t r = ((rows + 127) / 128 + 15) / 16 * 16;
    return (int)std::min<int64_t>(std::max<int64_t>(r, 64), 512);
}
__global__ __launch_bounds__(256) void key_norm_max_kernel(const uint16_t *k, int64_t ld, int64_t rows, int32_t heads,
                                                           int32_t per, uint32_t *kmax2) {
    const int t = threadIdx.x;
    const int c = (int)blockIdx.y * (kNormHeads * 16) + (t & 127);
    const int head = c >> 4;  // uniform over 16 consecutive lanes
    if (head >= heads) return;
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int nr = (int)min<int64_t>(per, rows - r0);
    const uint16_t *p = k + r0 * ld + 8 * c;
    float m = 0.f;
    int r = t >> 7;
    for (; r + 14 < nr; r += 16) {
        uint4 u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)(r + 2 * i) * ld);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[8];
            unpack8(u[i], f);
            float s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s2 = __builtin_fmaf(f[e], f[e], s2);
            m = fmaxf(m, sum16(s2));
        }
    }
    for (; r < nr; r += 2) {
        float f[8];
        unpack8(*reinterpret_cast<const uint4 *>(p + (int64_t)r * ld), f);
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 = __builtin_fmaf(f[e], f[e], s2);
        m = fmaxf(m, sum16(s2));
    }
    if ((t & 15) == 0) atomicMax(kmax2 + head, __float_as_uint(m));
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

// Combines the partial results of (head, tile) items cut into key-range
// pieces (at most 4, as the work schedule cuts them): per query row,
// o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) with M the largest m_s,
// rounded to BF16. Workgroup (item, quarter): 64 rows of one item, 16 rows at
// a time, 16 lanes per row with 8 channels each; every piece's loads of a row
// are issued before any of them is used.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float *part, int32_t records, int32_t pieces,
                                                         int32_t first, int32_t tiles_per_head, int64_t rows,
                                                         uint16_t *o, int64_t ld_o) {
    constexpr int kMaxPieces = 4;
    const int item = blockIdx.x;
    const int sub = threadIdx.x >> 4, cl = threadIdx.x & 15;
    const int hti = first + item;
    const int head = hti / tiles_per_head, tile = hti - head * tiles_per_head;
    const float2 *ml = reinterpret_cast<const float2 *>(part + (int64_t)records * BQ * D);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r = (int)blockIdx.y * 64 + it * 16 + sub;
        const int64_t q = (int64_t)tile * BQ + r;
        if (q >= rows) continue;
        float2 e[kMaxPieces];
        float4 v[kMaxPieces][2];
#pragma unroll
        for (int s = 0; s < kMaxPieces; ++s)
            if (s < pieces) {
                const int64_t rec = (int64_t)item * pieces + s;
                e[s] = ml[rec * BQ + r];
                const float4 *src = reinterpret_cast<const float4 *>(part + (rec * BQ + r) * D + 8 * cl);
                v[s][0] = src[0];
                v[s][1] = src[1];
            }
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int s = 0; s < kMaxPieces; ++s)
            if (s < pieces) M = fmaxf(M, e[s].x);
        float l = 0.f, a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMaxPieces; ++s)
            if (s < pieces) {
                const float w = __builtin_amdgcn_exp2f(e[s].x - M);
                l += w * e[s].y;
                a[0] += w * v[s][0].x; a[1] += w * v[s][0].y; a[2] += w * v[s][0].z; a[3] += w * v[s][0].w;
                a[4] += w * v[s][1].x; a[5] += w * v[s][1].y; a[6] += w * v[s][1].z; a[7] += w * v[s][1].w;
            }
        const float inv = 1.0f / l;
        *reinterpret_cast<uint4 *>(o + q * ld_o + head * D + 8 * cl) =
            make_uint4(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv),
                       pack_bf16x2(a[4] * inv, a[5] * inv), pack_bf16x2(a[6] * inv, a[7] * inv));
    }
}

// Transposed V of every segment of the plan into the workspace, and the
// largest squared key norm per head over all segments.
__global__ __launch_bounds__(64) void zero_u32_kernel(uint32_t *p, int32_t n) {
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Per-head maxima of a segment staged by h3_kv_stage merged into the call's.
__global__ __launch_bounds__(64) void kmax_merge_kernel(uint32_t *kmax2, const float *seg_kmax2, int32_t heads) {
    const int h = blockIdx.x * 64 + threadIdx.x;
    if (h < heads) atomicMax(kmax2 + h, __float_as_uint(seg_kmax2[h]));
}

void stage_vt(const VtPlan &plan, const uint16_t *k, int64_t ld_k, const uint16_t *v, int64_t ld_v, int32_t heads,
              uint8_t *ws, hipStream_t stream, const h3_qgroup *groups = nullptr, int32_t n_groups = 0) {
    if (plan.bytes == 0) return;
    uint32_t *kmax2 = reinterpret_cast<uint32_t *>(ws + plan.kmax_off);
    const int64_t kcols = (int64_t)(plan.bytes - plan.kmax_off) / 2;  // the 256-byte aligned area, as BF16 slots
    launch_zero_rows(reinterpret_cast<uint16_t *>(kmax2), kcols, kcols, 0, 1, stream);
    for (int gi = 0; gi < n_groups; ++gi)
        for (int s = 0; s < groups[gi].n_seg; ++s) {
            const h3_kv_seg &x = groups[gi].seg[s];
            if (x.k != nullptr && x.vt != nullptr)
                kmax_merge_kernel<<<dim3((unsigned)((heads + 63) / 64)), 64, 0, stream>>>(kmax2, x.kmax2, heads);
        }
    for (int i = 0; i < plan.n; ++i) {
        const VtSeg &e = plan.seg[i];
        const uint16_t *ks = e.own ? k + e.begin * ld_k : e.k + e.begin * e.ld;
        const int per = norm_rows_per_wg(e.len);
        key_norm_max_kernel<<<dim3((unsigned)((e.len + per - 1) / per), (unsigned)((heads + kNormHeads - 1) / kNormHeads)),
                              256, 0, stream>>>(
            ks, e.own ? ld_k : e.ld, e.len, heads, per, kmax2);
    }
    for (int i = 0; i < plan.n; ++i) {
        const VtSeg &e = plan.seg[i];
        const uint16_t *src = e.own ? v + e.begin * ld_v : e.v + e.begin * e.ld;
        const int64_t ld = e.own ? ld_v : e.ld;
        vt_transpose_kernel<<<dim3((unsigned)(e.lpad / BKV), (unsigned)heads), 256, 0, stream>>>(
            src, ld, e.len, reinterpret_cast<uint16_t *>(ws + e.off), e.lpad);
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
        dense.seg[0] = h3_kv_seg{nullptr, nullptr, 0, 0, valid_len, nullptr, nullptr};
        groups = &dense;
        n_groups = valid_len > 0 ? 1 : 0;
    }
    // Stage V^T once per distinct segment.
    VtPlan plan;
    vt_plan(is_dense ? nullptr : groups, is_dense ? 0 : n_groups, valid_len, heads, &plan);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    stage_vt(plan, k, ld_k, v, ld_v, heads, ws, stream, is_dense ? nullptr : groups, is_dense ? 0 : n_groups);
    std::pair<int64_t, int64_t> cov[H3_MAX_GROUPS];
    int nc = 0;
    for (int gi = 0; gi < n_groups; ++gi)
        if (groups[gi].q_end > groups[gi].q_begin) cov[nc++] = {groups[gi].q_begin, groups[gi].q_end};
    AttnSchedule sch;
    attn_schedule(is_dense ? nullptr : groups, is_dense ? 0 : n_groups, valid_len, heads, &sch);
    AttnArgs a = {};
    a.ld_q = ld_q;
    a.ld_o = ld_o;
    a.heads = heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.kmax2 = reinterpret_cast<const float *>(ws + plan.kmax_off);
    a.flags = reinterpret_cast<int32_t *>(ws + plan.flags_off);
    a.queue = reinterpret_cast<int32_t *>(ws + plan.queue_off);
    a.n_items = sch.items;
    const AttnDeal deal = attn_deal(sch.items);
    a.static_tickets = deal.static_tickets;
    a.part = reinterpret_cast<float *>(ws + plan.part_off);
    a.part_records = sch.split_items * sch.pieces;
    a.n_ranges = sch.n;
    for (int gi = 0; gi < n_groups; ++gi) {
        const h3_qgroup &g = groups[gi];
        if (g.q_end <= g.q_begin) continue;
        AttnGroup &G = a.grp[gi];
        G.q = q + g.q_begin * ld_q;
        G.o = o + g.q_begin * ld_o;
        G.rows = g.q_end - g.q_begin;
        G.tiles_per_head = (int32_t)((G.rows + BQ - 1) / BQ);
        G.n_seg = g.n_seg;
        for (int s = 0; s < g.n_seg; ++s) {
            const h3_kv_seg &ss = g.seg[s];
            if (ss.k != nullptr && ss.vt != nullptr) {  // staged by h3_kv_stage
                G.sk[s] = ss.k + ss.begin * ss.ld;
                G.sldk[s] = ss.ld;
                G.svt[s] = ss.vt;
                G.slpad[s] = (ss.len + 63) / 64 * 64;
                G.slen[s] = ss.len;
                continue;
            }
            const VtSeg &e = plan.seg[plan.map[gi][s]];
            if (ss.k == nullptr) {
                G.sk[s] = k + ss.begin * ld_k;
                G.sldk[s] = ld_k;
            } else {
                G.sk[s] = ss.k + ss.begin * ss.ld;
                G.sldk[s] = ss.ld;
            }
            G.svt[s] = reinterpret_cast<const uint16_t *>(ws + e.off);
            G.slpad[s] = e.lpad;
            G.slen[s] = ss.len;
        }
    }
    int split_range = -1;
    for (int i = 0; i < sch.n; ++i) {
        a.rng_end[i] = sch.end[i];
        a.rng_group[i] = sch.group[i];
        a.rng_first[i] = sch.first[i];
        a.rng_count[i] = sch.count[i];
        a.rng_split[i] = sch.split[i];
        if (sch.split[i] > 1) split_range = i;
    }
    const dim3 grid((unsigned)deal.grid);
    if (sch.n == 1 && split_range < 0 && sch.group[0] != 0) {  // the single-range kernel reads grp[0]
        a.grp[0] = a.grp[sch.group[0]];
        a.rng_group[0] = 0;
    }
    if (sch.n > 1 || split_range >= 0) {
        launch_attention_fixed_multi(grid, a, stream);
        attention_fwd_kernel<false, false, true><<<grid, kThreads, 0, stream>>>(a);
    } else if (sch.n == 1) {
        launch_attention_fixed(false, grid, a, stream);
        attention_fwd_kernel<false, false, false><<<grid, kThreads, 0, stream>>>(a);
    }
    if (split_range >= 0) {
        const AttnGroup &G = a.grp[sch.group[split_range]];
        attn_merge_kernel<<<dim3((unsigned)sch.split_items, BQ / 64), 256, 0, stream>>>(
            a.part, a.part_records, sch.pieces, sch.first[split_range], G.tiles_per_head, G.rows, G.o, ld_o);
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

// SolarWM H3 Realtime, stage 3: an external K/V segment staged once (V^T plane
// and per-head key norm maxima, the same kernels attention stages with) for
// the attention calls that read it.
extern "C" int h3_kv_stage(const uint16_t *k, const uint16_t *v, int64_t ld, int64_t len, int32_t heads,
                           int32_t head_dim, uint16_t *vt, float *kmax2, void *stream) {
    int s = h3_check_kv_stage(k, v, ld, len, heads, head_dim, vt, kmax2);
    if (s != H3_OK || len == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    const int64_t lpad = (len + 63) / 64 * 64;
    uint32_t *km = reinterpret_cast<uint32_t *>(kmax2);
    zero_u32_kernel<<<dim3((unsigned)((heads + 63) / 64)), 64, 0, st>>>(km, heads);
    const int per = norm_rows_per_wg(len);
    key_norm_max_kernel<<<dim3((unsigned)((len + per - 1) / per), (unsigned)((heads + kNormHeads - 1) / kNormHeads)), 256,
                          0, st>>>(k, ld, len, heads, per, km);
    vt_transpose_kernel<<<dim3((unsigned)(lpad / BKV), (unsigned)heads), 256, 0, st>>>(v, ld, len, vt, lpad);
    return launch_status();
}

// ---------------------------------------------------------------------------
// h3_attention_noalloc: h3_attention with its workspace in a fixed device array
// of this library instead of a caller buffer, for callers that cannot allocate.
// The array has static storage: every GPU the library runs on holds its own
// copy until the process ends. Host code only ever uses the device address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in there). The kernels need nothing cleared in it: the
// key-norm maxima are zeroed by a fill kernel inside the call, the V^T planes,
// partial records and workgroup flags are written before they are read.
// ---------------------------------------------------------------------------
namespace h3 {
namespace {

static __device__ __align__(256) uint8_t scratch[H3_ATTENTION_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kScratchDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        std::fprintf(stderr, "libh3block: hipGetDevice failed: %s (%d)\n", hipGetErrorString(e), (int)e);
        return H3_ERR_HIP;
    }
    if (dev < 0 || dev >= kScratchDevices) return H3_ERR_DEVICE;
    uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (a == 0) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            std::fprintf(stderr, "libh3block: hipGetSymbolAddress(scratch) failed: %s (%d)\n",
                         hipGetErrorString(e), (int)e);
            return H3_ERR_HIP;
        }
        a = reinterpret_cast<uintptr_t>(p);
        g_scratch_addr[dev].store(a, std::memory_order_release);
    }
    *out = reinterpret_cast<void *>(a);
    return H3_OK;
}

}  // namespace
}  // namespace h3

extern "C" int h3_attention_noalloc(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                                    const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf,
                                    int64_t valid_len, int32_t heads, int32_t head_dim, float softmax_scale,
                                    const h3_qgroup *groups, int32_t n_groups, void *stream) {
    // Every check but the workspace's first (no workspace given yet), then the
    // size limit, then the full check against the device array.
    int s = h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim,
                               softmax_scale, groups, n_groups, nullptr, 0);
    if (s != H3_OK && s != H3_ERR_WORKSPACE) return s;
    if (L_buf == 0) return H3_OK;
    if (h3_attention_workspace_bytes(valid_len, heads, groups, n_groups) > (size_t)H3_ATTENTION_SCRATCH_BYTES)
        return H3_ERR_WORKSPACE;
    if ((s = device_check()) != H3_OK) return s;
    void *ws = nullptr;
    if ((s = scratch_address(&ws)) != H3_OK) return s;
    s = h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim, softmax_scale,
                           groups, n_groups, ws, (size_t)H3_ATTENTION_SCRATCH_BYTES);
    if (s != H3_OK) return s;
    launch_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, softmax_scale, groups, n_groups,
                     ws, (hipStream_t)stream);
    return launch_status();
}

namespace h3 {

void launch_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                             int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len,
                             int64_t prefix_len, int32_t heads, float softmax_scale, const uint16_t *blocks,
                             const int32_t *counts, void *workspace, hipStream_t stream) {
    if (prefix_len >= valid_len) {  // no target rows: dense attention
        launch_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, softmax_scale, nullptr, 0,
                         workspace, stream);
        return;
    }
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    h3_qgroup g;
    sparse_vt_group(valid_len, prefix_len, &g);
    VtPlan plan;
    vt_plan(&g, 1, valid_len, heads, &plan);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    stage_vt(plan, k, ld_k, v, ld_v, heads, ws, stream);
    const int64_t T = valid_len - prefix_len;
    AttnArgs a = {};
    AttnGroup &G = a.grp[0];
    G.q = q;
    G.o = o;
    a.ld_q = ld_q;
    a.ld_o = ld_o;
    G.rows = valid_len;
    a.heads = heads;
    G.tiles_per_head = (int32_t)((T + BQ - 1) / BQ);
    G.n_seg = 2;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.kmax2 = reinterpret_cast<const float *>(ws + plan.kmax_off);
    a.flags = reinterpret_cast<int32_t *>(ws + plan.flags_off);
    a.queue = reinterpret_cast<int32_t *>(ws + plan.queue_off);
    for (int s = 0; s < 2; ++s) {
        const VtSeg &e = plan.seg[plan.map[0][s]];
        G.sk[s] = k + g.seg[s].begin * ld_k;
        G.sldk[s] = ld_k;
        G.svt[s] = reinterpret_cast<const uint16_t *>(ws + e.off);
        G.slpad[s] = e.lpad;
        G.slen[s] = g.seg[s].len;
    }
    a.blocks = blocks;
    a.counts = counts;
    a.n_kb = (int32_t)((T + BKV - 1) / BKV);
    a.pre_tiles = (int32_t)((prefix_len + BQ - 1) / BQ);
    a.pre_items = (heads * a.pre_tiles + 7) / 8 * 8;
    a.n_ranges = 1;
    a.rng_split[0] = 1;
    a.prefix_len = prefix_len;
    a.tgt_rows = T;
    a.n_items = a.pre_items + G.tiles_per_head * heads;
    a.rng_end[0] = a.n_items;
    const AttnDeal deal = attn_deal(a.n_items);
    a.static_tickets = deal.static_tickets;
    const unsigned grid = (unsigned)deal.grid;
    launch_attention_fixed(true, dim3(grid), a, stream);
    attention_fwd_kernel<true, false, false><<<dim3(grid), kThreads, 0, stream>>>(a);
    launch_zero_rows(o, ld_o, (int64_t)heads * D, valid_len, L_buf, stream);
}

}  // namespace h3

extern "C" int h3_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                                   const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf,
                                   int64_t valid_len, int64_t prefix_len, int32_t heads, int32_t head_dim,
                                   float softmax_scale, const uint16_t *blocks, const int32_t *counts,
                                   void *workspace, size_t ws_bytes, void *stream) {
    int s = h3_check_sparse_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, prefix_len, heads,
                                      head_dim, softmax_scale, blocks, counts, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_sparse_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, prefix_len, heads, softmax_scale,
                            blocks, counts, workspace, (hipStream_t)stream);
    return launch_status();
}
