// Host-only argument validation for every entry point of libh3block.
//
// No HIP header is included: these checks run before anything is launched
// (a call that fails here writes nothing) and are callable on a machine
// without a GPU. Fail-closed rejection of unsupported configurations follows
// the Sol-H3 report (Appendix B, "Implementation scope": unsupported
// configurations are rejected before installation).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <queue>
#include <vector>

#include "h3_internal.h"

namespace h3 {
namespace {

constexpr int64_t kBf16 = 2;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A strided matrix in memory: `rows` rows of `cols` elements, row stride `ld`.
struct Mat {
    uintptr_t base;
    int64_t rows, cols, ld, elem;
    bool empty() const { return base == 0 || rows <= 0 || cols <= 0; }
    uintptr_t end() const { return base + (uintptr_t)(((rows - 1) * ld + cols) * elem); }
};

Mat mat(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t elem = kBf16) {
    return Mat{reinterpret_cast<uintptr_t>(p), rows, cols, ld, elem};
}

// Byte span of a small device array (lists, counts, workspace).
Mat bytes_of(const void *p, int64_t n) { return mat(p, 1, n, n, 1); }

// True when two strided matrices can share a byte. Matrices with the same
// row stride are compared column-block-wise (column blocks of one packed
// buffer are disjoint); otherwise their spans are compared.
bool overlap(const Mat &a, const Mat &b) {
    if (a.empty() || b.empty()) return false;
    if (a.end() <= b.base || b.end() <= a.base) return false;
    if (a.ld == b.ld && a.elem == b.elem) {
        const int64_t rowb = a.ld * a.elem;
        const int64_t diff = (int64_t)b.base - (int64_t)a.base;
        int64_t c = diff % rowb;
        if (c < 0) c += rowb;
        const int64_t wa = a.cols * a.elem, wb = b.cols * b.elem;
        // b's columns start c bytes into a row of a (or c - rowb, wrapping)
        const bool hit1 = c < wa && c + wb > 0;
        const bool hit2 = (c - rowb) < wa && (c - rowb) + wb > 0;
        return hit1 || hit2;
    }
    return true;
}

bool same(const Mat &a, const Mat &b) { return a.base == b.base && a.ld == b.ld; }

int check_rows(int64_t L_buf, int64_t valid_len) {
    if (L_buf < 0 || valid_len < 0 || valid_len > L_buf) return H3_ERR_SHAPE;
    return H3_OK;
}

int check_bf16_mat(const void *p, int64_t ld, int64_t cols, bool required = true) {
    if (p == nullptr) return required ? H3_ERR_NULL : H3_OK;
    if (ld < cols) return H3_ERR_SHAPE;
    if (!aligned16(p) || (ld % 8) != 0) return H3_ERR_ALIGN;
    return H3_OK;
}

#define H3_TRY(expr)                 \
    do {                             \
        int _s = (expr);             \
        if (_s != H3_OK) return _s;  \
    } while (0)

}  // namespace

int check_dims(const h3_dims *d) {
    if (d == nullptr) return H3_ERR_NULL;
    if (d->heads <= 0 || d->head_dim <= 0 || d->hidden <= 0 || d->ffn <= 0) return H3_ERR_SHAPE;
    if ((int64_t)d->heads * d->head_dim != d->hidden) return H3_ERR_SHAPE;
    if (d->head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
    if (d->hidden > kMaxHidden) return H3_ERR_UNSUPPORTED;
    if (d->ffn % 64 != 0) return H3_ERR_UNSUPPORTED;  // FFN-down reduction runs in K steps of 64
    if (d->rot_dim < 0 || d->rot_dim > d->head_dim || d->rot_dim % 16 != 0) return H3_ERR_UNSUPPORTED;
    if (d->norm_type != 0 && d->norm_type != 1) return H3_ERR_UNSUPPORTED;
    if (d->rope_pairing != 0 && d->rope_pairing != 1) return H3_ERR_UNSUPPORTED;
    if (d->reserved != 0) return H3_ERR_SHAPE;
    if (!(d->eps >= 0.0f) || !std::isfinite(d->eps)) return H3_ERR_SHAPE;
    if (!(d->rope_theta > 0.0f) || !std::isfinite(d->rope_theta)) return H3_ERR_SHAPE;
    return H3_OK;
}

void sparse_geometry(int64_t valid_len, int64_t prefix_len, int32_t heads, SparseGeom *g) {
    const int64_t T = valid_len > prefix_len ? valid_len - prefix_len : 0;
    g->T = T;
    g->n_qb = (T + H3_SPARSE_Q_BLOCK - 1) / H3_SPARSE_Q_BLOCK;
    g->n_kb = (T + H3_SPARSE_K_BLOCK - 1) / H3_SPARSE_K_BLOCK;
    int64_t per = (g->n_kb + 255) / 256;
    per = (per + 3) / 4 * 4;
    g->per = per;
    g->n_kb_pad = 256 * per;
    g->qbar_off = 0;
    const int64_t qbar_bytes = (int64_t)heads * g->n_qb * kHeadDim * 4;
    g->kbar_off = (qbar_bytes + kWsAlign - 1) / kWsAlign * kWsAlign;
    g->ws_bytes = (size_t)(g->kbar_off + (int64_t)heads * kHeadDim * g->n_kb_pad * 4);
}

void sparse_vt_group(int64_t valid_len, int64_t prefix_len, h3_qgroup *g) {
    std::memset(g, 0, sizeof(*g));
    g->q_begin = 0;
    g->q_end = valid_len;
    g->n_seg = 2;
    g->seg[0] = h3_kv_seg{nullptr, nullptr, 0, 0, prefix_len, nullptr, nullptr};
    g->seg[1] = h3_kv_seg{nullptr, nullptr, 0, prefix_len, valid_len - prefix_len, nullptr, nullptr};
}

// Finish time of list scheduling on kAttnSlots identical workgroup slots, all
// free at time 0: each unit (a length in key tiles) goes, in order, to the
// slot that frees first. This is how the dispatcher hands out a launch's
// workgroups once its full rounds are done.
static int64_t list_makespan(const std::vector<int64_t> &units) {
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
    for (int i = 0; i < kAttnSlots; ++i) free_at.push(0);
    int64_t end = 0;
    for (const int64_t u : units) {
        const int64_t t = free_at.top() + u;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
    }
    return end;
}

void attn_schedule(const h3_qgroup *groups, int n_groups, int64_t dense_len, int heads, AttnSchedule *out) {
    std::memset(out, 0, sizeof(*out));
    int order[H3_MAX_GROUPS];
    int64_t rows[H3_MAX_GROUPS], kt[H3_MAX_GROUPS];
    int nc = 0;
    if (groups == nullptr) {
        if (dense_len > 0) {
            rows[0] = dense_len;
            kt[0] = (dense_len + 63) / 64;
            order[nc++] = 0;
        }
    } else {
        for (int g = 0; g < n_groups && g < H3_MAX_GROUPS; ++g) {
            rows[g] = groups[g].q_end - groups[g].q_begin;
            if (rows[g] <= 0) continue;
            kt[g] = 0;
            for (int s = 0; s < groups[g].n_seg && s < H3_MAX_SEGMENTS; ++s)
                kt[g] += (std::max<int64_t>(groups[g].seg[s].len, 0) + 63) / 64;
            order[nc++] = g;
        }
    }
    std::stable_sort(order, order + nc, [&](int x, int y) { return kt[x] > kt[y]; });
    auto add = [&](int g, int32_t first, int32_t count, int32_t split) {
        out->group[out->n] = g;
        out->first[out->n] = first;
        out->count[out->n] = count;
        out->split[out->n] = split;
        ++out->n;
    };
    for (int oi = 0; oi < nc; ++oi) {
        const int g = order[oi];
        const int32_t n = (int32_t)((rows[g] + 255) / 256) * heads;
        int32_t pieces = 1, full = n;
        if (oi == 0 && n < 4 * kAttnSlots) {
            full = n / kAttnSlots * kAttnSlots;
            const int32_t tail = n - full;
            if (tail > 0) {
                // The piece count p (1-4) whose tail finishes soonest: list
                // scheduling of the tail's pieces, then the other groups'
                // items (longest group first, as they are dispatched), each
                // unit costing its key tiles plus kAttnItemTiles for the
                // item's fixed work. Each piece keeps at least 4 key tiles,
                // and the tail's pieces stay under 512 partial records.
                std::vector<int64_t> rest;
                for (int oj = 1; oj < nc && (int64_t)rest.size() < kAttnSimUnits; ++oj) {
                    const int64_t cnt = (rows[order[oj]] + 255) / 256 * heads;
                    for (int64_t i = 0; i < cnt && (int64_t)rest.size() < kAttnSimUnits; ++i)
                        rest.push_back(kt[order[oj]] + kAttnItemTiles);
                }
                int64_t best = -1;
                for (int32_t p = 1; p <= 4; ++p) {
                    if (p > 1 && ((int64_t)tail * p > 511 || kt[g] / p < 4)) break;
                    std::vector<int64_t> units;
                    units.reserve((size_t)tail * p + rest.size());
                    for (int32_t i = 0; i < tail; ++i)
                        for (int32_t q = 0; q < p; ++q)
                            units.push_back((q + 1) * kt[g] / p - q * kt[g] / p + kAttnItemTiles);
                    units.insert(units.end(), rest.begin(), rest.end());
                    const int64_t t = list_makespan(units);
                    if (best < 0 || t < best) {
                        best = t;
                        pieces = p;
                    }
                }
                if (pieces < 2) full = n;
            }
        }
        if (full > 0) add(g, 0, full, 1);
        if (pieces > 1) {
            add(g, full, n - full, pieces);
            out->split_items = n - full;
            out->pieces = pieces;
        }
    }
    int32_t items = 0;
    const bool multi = out->n > 1 || out->pieces > 1;
    for (int i = 0; i < out->n; ++i) {
        const int32_t c = out->count[i] * out->split[i];
        items += multi ? (c + 7) / 8 * 8 : c;
        out->end[i] = items;
    }
    out->items = items;
}

// The stream-K split of the last round, if it pays.
static void gemm_plan_tail(GemmPlan &g) {
    const int32_t tail = g.tiles % kGemmSlots;
    if (tail == 0 || 5 * tail > 4 * kGemmSlots) return;
    // The split costs about as much as 55 stages of the last round (the
    // partial sums' traffic, the fix-up pass, two more launches; measured on
    // the block's projections at 4,096 and 5,424 rows): take it only where the
    // idle share of the last round is worth more.
    if ((int64_t)g.stages * (kGemmSlots - tail) < (int64_t)kSkWorthStages * kGemmSlots) return;
    const int64_t units = (int64_t)tail * g.stages;
    const int32_t groups = (int32_t)std::min<int64_t>(kGemmSlots, units / kSkMinStages);
    if (groups <= tail) return;  // no range would be shorter than a tile
    g.dp_tiles = g.tiles - tail;
    g.sk_tiles = tail;
    g.sk_groups = groups;
    g.part_bytes = (size_t)groups * 2 * 256 * 256 * 4;
}

GemmPlan gemm_plan(int64_t M_valid, int64_t N, int64_t K, int32_t epilogue) {
    GemmPlan g = {};
    g.tiles_m = (int32_t)((std::max<int64_t>(M_valid, 0) + 255) / 256);
    g.tiles_n = epilogue == H3_EPI_SWIGLU ? (int32_t)((N / 2 + 127) / 128) : (int32_t)((N + 255) / 256);
    g.tiles = g.tiles_m * g.tiles_n;
    g.stages = (int32_t)(K / 64);
    g.dp_tiles = g.tiles;
    gemm_plan_tail(g);
    g.ws_bytes = g.part_bytes;
    if (g.dp_tiles >= kGemmDealRounds * kGemmSlots) {
        const int32_t T = g.dp_tiles / 8, W = std::max(3 * kGemmSlots / 8, T / 12);
        g.deal = true;
        g.static_tickets = T - W;
        g.grid = 8 * (g.static_tickets + W + W / 2);
        g.queue_off = (g.part_bytes + 255) / 256 * 256;
        g.ws_bytes = g.queue_off + 256;
    }
    return g;
}

size_t gemm_ws_bytes_max(int64_t M_buf, int64_t N, int64_t K, int32_t epilogue) {
    // The partial sums grow with the tail's units (at most kGemmSlots ranges)
    // and need not grow with M: take the plan of every tile count up to M_buf's.
    const int64_t tm_max = (std::max<int64_t>(M_buf, 0) + 255) / 256;
    size_t best = 0;
    for (int64_t tm = 1; tm <= tm_max; ++tm) best = std::max(best, gemm_plan(tm * 256, N, K, epilogue).ws_bytes);
    return best;
}

void vt_plan(const h3_qgroup *groups, int n_groups, int64_t dense_len, int heads, VtPlan *out) {
    out->n = 0;
    out->bytes = 0;
    out->kmax_off = 0;
    auto add = [&](int own, const uint16_t *k, const uint16_t *v, int64_t ld, int64_t begin, int64_t len) {
        for (int i = 0; i < out->n; ++i) {
            const VtSeg &e = out->seg[i];
            if (e.own == own && e.v == v && e.ld == ld && e.begin == begin && e.len == len) return i;
        }
        VtSeg &e = out->seg[out->n];
        e.own = own; e.k = k; e.v = v; e.ld = ld; e.begin = begin; e.len = len;
        e.lpad = (len + 63) / 64 * 64;
        e.off = (int64_t)out->bytes;
        out->bytes += (size_t)heads * kHeadDim * e.lpad * 2;
        return out->n++;
    };
    int64_t qtiles = 0;  // 256-row query tiles over all groups
    int n_launch_groups = 1;
    bool staged = false;  // a segment staged by h3_kv_stage (no plane here)
    if (groups == nullptr) {
        if (dense_len > 0) out->map[0][0] = add(1, nullptr, nullptr, 0, 0, dense_len);
        qtiles = (dense_len + 255) / 256;
    } else {
        n_launch_groups = std::max(1, std::min(n_groups, H3_MAX_GROUPS));
        for (int g = 0; g < n_groups && g < H3_MAX_GROUPS; ++g) {
            qtiles += (std::max<int64_t>(groups[g].q_end - groups[g].q_begin, 0) + 255) / 256;
            for (int s = 0; s < groups[g].n_seg && s < H3_MAX_SEGMENTS; ++s) {
                const h3_kv_seg &x = groups[g].seg[s];
                if (x.k != nullptr && x.vt != nullptr) {
                    out->map[g][s] = -1;  // staged by h3_kv_stage: read in place
                    staged = true;
                    continue;
                }
                out->map[g][s] = x.k == nullptr ? add(1, nullptr, nullptr, 0, x.begin, x.len)
                                                : add(0, x.k, x.v, x.ld, x.begin, x.len);
            }
        }
    }
    out->flags_off = 0;
    out->part_off = 0;
    out->queue_off = 0;
    if (out->n > 0 || staged) {
        auto align = [](size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; };
        // Partial results of the items cut into pieces: a partial round has
        // fewer than 256 items, cut into at most 4 pieces each and fewer than
        // 512 records of 256 rows in all. Reserved from the row count alone so that the size never
        // shrinks as rows grow (a dense plan for the buffer rows also fits
        // any valid length below them).
        const int64_t records = std::min<int64_t>(511, 4 * qtiles * heads);
        out->part_off = (int64_t)out->bytes;
        out->bytes += align((size_t)records * 256 * (kHeadDim + 2) * 4);
        out->kmax_off = (int64_t)out->bytes;
        out->bytes += align((size_t)heads * 4);
        // workgroups of the launch: query tiles of 256 rows per head and group,
        // plus the block-sparse launch's split of the rows into prefix and
        // target tiles (at most one more tile per head)
        // (pieces add fewer than 512 items; every range may be padded by 7)
        out->flags_off = (int64_t)out->bytes;
        out->bytes += align((size_t)((qtiles + 1) * heads + 8 * (n_launch_groups + 1) + 512) * 4);
        out->queue_off = (int64_t)out->bytes;
        out->bytes += align((size_t)kAttnQueueWords * 4);
    }
}

// Partial-sum area for the block's four projections (run one after another).
static size_t block_gemm_part_bytes(const h3_dims *d, int64_t L_buf) {
    const int64_t H = d->hidden, F = d->ffn;
    return std::max({gemm_ws_bytes_max(L_buf, 3 * H, H, H3_EPI_STORE),
                     gemm_ws_bytes_max(L_buf, H, H, H3_EPI_RESIDUAL),
                     gemm_ws_bytes_max(L_buf, 2 * F, H, H3_EPI_SWIGLU),
                     gemm_ws_bytes_max(L_buf, H, F, H3_EPI_RESIDUAL)});
}

bool ws_layout(const h3_dims *d, int64_t L_buf, const h3_qgroup *groups, int n_groups, WsLayout *out) {
    if (check_dims(d) != H3_OK || L_buf < 0) return false;
    if (groups != nullptr && (n_groups < 1 || n_groups > H3_MAX_GROUPS)) return false;
    const int64_t H = d->hidden, F = d->ffn;
    const int64_t cols[H3_WS_VT] = {H, 3 * H, H, H, H, F};
    int64_t off = 0;
    auto align = [](int64_t b) { return (b + (int64_t)kWsAlign - 1) / (int64_t)kWsAlign * (int64_t)kWsAlign; };
    for (int i = 0; i < H3_WS_VT; ++i) {
        out->off[i] = off;
        out->ld[i] = cols[i];
        out->cols[i] = cols[i];
        off += align(L_buf * cols[i] * kBf16);
    }
    VtPlan p;
    vt_plan(groups, n_groups, L_buf, d->heads, &p);
    out->off[H3_WS_VT] = off;
    out->ld[H3_WS_VT] = (int64_t)p.bytes;
    out->cols[H3_WS_VT] = 0;
    off += align((int64_t)p.bytes);
    const int64_t part = (int64_t)block_gemm_part_bytes(d, L_buf);
    out->off[H3_WS_GEMM] = off;
    out->ld[H3_WS_GEMM] = part;
    out->cols[H3_WS_GEMM] = 0;
    off += align(part);
    out->total = (size_t)off;
    return true;
}

bool block_sparse_layout(const h3_dims *d, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                         BlockSparseLayout *out) {
    if (!ws_layout(d, L_buf, nullptr, 0, &out->base)) return false;
    if (valid_len < 0 || valid_len > L_buf || prefix_len < 0 || prefix_len > valid_len) return false;
    auto align = [](int64_t b) { return (b + (int64_t)kWsAlign - 1) / (int64_t)kWsAlign * (int64_t)kWsAlign; };
    WsLayout &l = out->base;
    int64_t vt = l.ld[H3_WS_VT];
    if (valid_len > prefix_len) {
        h3_qgroup g;
        sparse_vt_group(valid_len, prefix_len, &g);
        VtPlan p;
        vt_plan(&g, 1, valid_len, d->heads, &p);
        vt = std::max<int64_t>(vt, (int64_t)p.bytes);
    }
    l.ld[H3_WS_VT] = vt;
    int64_t off = l.off[H3_WS_VT] + align(vt);
    l.off[H3_WS_GEMM] = off;
    off += align(l.ld[H3_WS_GEMM]);
    l.total = (size_t)off;
    SparseGeom g;
    sparse_geometry(valid_len, prefix_len, d->heads, &g);
    out->blocks_off = off;
    off += align((int64_t)d->heads * g.n_qb * g.n_kb * 2);
    out->counts_off = off;
    off += align((int64_t)d->heads * g.n_qb * 4);
    out->select_off = off;
    off += align(g.T > 0 ? (int64_t)g.ws_bytes : 0);
    out->total = (size_t)off;
    return true;
}

bool mx_ws_layout(const h3_dims *d, int64_t L_buf, int64_t valid_len, int64_t prefix_len, MxWsLayout *out) {
    if (check_dims(d) != H3_OK || L_buf < 0) return false;
    if (d->hidden % 128 != 0 || d->ffn % 128 != 0) return false;
    if (valid_len < 0 || valid_len > L_buf) return false;
    const int64_t H = d->hidden, F = d->ffn;
    auto align = [](int64_t b) { return (b + (int64_t)kWsAlign - 1) / (int64_t)kWsAlign * (int64_t)kWsAlign; };
    VtPlan p;
    vt_plan(nullptr, 0, L_buf, d->heads, &p);
    int64_t vt = (int64_t)p.bytes;
    const bool sparse = prefix_len >= 0 && prefix_len < valid_len;
    SparseGeom g = {};
    if (sparse) {
        h3_qgroup grp;
        sparse_vt_group(valid_len, prefix_len, &grp);
        VtPlan ps;
        vt_plan(&grp, 1, valid_len, d->heads, &ps);
        vt = std::max<int64_t>(vt, (int64_t)ps.bytes);
        sparse_geometry(valid_len, prefix_len, d->heads, &g);
    }
    const int64_t bytes[H3_MXWS_COUNT] = {L_buf * H,      L_buf * H / 32, L_buf * 3 * H * 2, L_buf * H * 2,
                                          L_buf * H,      L_buf * H / 32, L_buf * H * 2,     L_buf * H,
                                          L_buf * H / 32, L_buf * F,      L_buf * F / 32,    vt,
                                          sparse ? (int64_t)d->heads * g.n_qb * g.n_kb * 2 : 0,
                                          sparse ? (int64_t)d->heads * g.n_qb * 4 : 0,
                                          sparse ? (int64_t)g.ws_bytes : 0};
    int64_t off = 0;
    for (int i = 0; i < H3_MXWS_COUNT; ++i) {
        out->off[i] = off;
        off += align(bytes[i]);
    }
    out->total = (size_t)off;
    return true;
}

}  // namespace h3

using namespace h3;

extern "C" {

const char *h3_status_string(int s) {
    switch (s) {
        case H3_OK: return "H3_OK";
        case H3_ERR_NULL: return "H3_ERR_NULL: a required pointer is NULL";
        case H3_ERR_SHAPE: return "H3_ERR_SHAPE: sizes inconsistent or out of range";
        case H3_ERR_UNSUPPORTED: return "H3_ERR_UNSUPPORTED: configuration not implemented";
        case H3_ERR_ALIGN: return "H3_ERR_ALIGN: pointer not 16-byte aligned or stride not a multiple of 8";
        case H3_ERR_ALIAS: return "H3_ERR_ALIAS: buffers overlap";
        case H3_ERR_WORKSPACE: return "H3_ERR_WORKSPACE: workspace missing or too small";
        case H3_ERR_DEVICE: return "H3_ERR_DEVICE: current device is not gfx950";
        case H3_ERR_HIP: return "H3_ERR_HIP: a HIP runtime call failed";
        default: return "unknown h3 status";
    }
}

int h3_abi_version(void) { return H3_ABI_VERSION; }

size_t h3_block_workspace_bytes(const h3_dims *dims, int64_t L_buf, const h3_qgroup *groups, int32_t n_groups) {
    WsLayout l;
    if (!ws_layout(dims, L_buf, groups, n_groups, &l)) return 0;
    return l.total;
}

size_t h3_attention_workspace_bytes(int64_t valid_len, int32_t heads, const h3_qgroup *groups,
                                    int32_t n_groups) {
    if (valid_len < 0 || heads <= 0) return 0;
    if (groups != nullptr && (n_groups < 1 || n_groups > H3_MAX_GROUPS)) return 0;
    VtPlan p;
    vt_plan(groups, n_groups, valid_len, heads, &p);
    return p.bytes;
}

size_t h3_block_sparse_workspace_bytes(const h3_dims *dims, int64_t L_buf, int64_t valid_len,
                                       int64_t prefix_len) {
    BlockSparseLayout l;
    if (!block_sparse_layout(dims, L_buf, valid_len, prefix_len, &l)) return 0;
    return l.total;
}

int h3_block_sparse_workspace_layout(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                     int64_t *blocks_off, int64_t *counts_off) {
    if (blocks_off == nullptr || counts_off == nullptr) return H3_ERR_NULL;
    BlockSparseLayout l;
    if (!block_sparse_layout(dims, L_buf, valid_len, prefix_len, &l)) return H3_ERR_SHAPE;
    *blocks_off = l.blocks_off;
    *counts_off = l.counts_off;
    return H3_OK;
}

size_t h3_sparse_attention_workspace_bytes(int64_t valid_len, int64_t prefix_len, int32_t heads) {
    if (valid_len < 0 || prefix_len < 0 || prefix_len > valid_len || heads <= 0) return 0;
    if (prefix_len == valid_len) return h3_attention_workspace_bytes(valid_len, heads, nullptr, 0);
    h3_qgroup g;
    sparse_vt_group(valid_len, prefix_len, &g);
    return h3_attention_workspace_bytes(valid_len, heads, &g, 1);
}

int h3_block_workspace_layout(const h3_dims *dims, int64_t L_buf, const h3_qgroup *groups, int32_t n_groups,
                              int64_t offsets[H3_WS_COUNT], int64_t lds[H3_WS_COUNT]) {
    if (offsets == nullptr || lds == nullptr) return H3_ERR_NULL;
    H3_TRY(check_dims(dims));
    if (L_buf < 0) return H3_ERR_SHAPE;
    WsLayout l;
    if (!ws_layout(dims, L_buf, groups, n_groups, &l)) return H3_ERR_SHAPE;
    for (int i = 0; i < H3_WS_COUNT; ++i) {
        offsets[i] = l.off[i];
        lds[i] = l.ld[i];
    }
    return H3_OK;
}

int h3_check_fused_modulate_norm(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                 const float *shift, const float *scale, const float *gate,
                                 int64_t ld_mod_group, int32_t n_mod_groups, const uint16_t *x1_out,
                                 int64_t ld_x1, const uint16_t *h_out, int64_t ld_h, int64_t L_buf,
                                 int64_t valid_len, int32_t hidden, float eps, int32_t norm_type) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (hidden <= 0) return H3_ERR_SHAPE;
    if (hidden > kMaxHidden) return H3_ERR_UNSUPPORTED;
    if (hidden % 8 != 0) return H3_ERR_ALIGN;
    if (norm_type != 0 && norm_type != 1) return H3_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    if (!x || !h_out || !shift || !scale) return H3_ERR_NULL;
    if (branch && (!gate || !x1_out)) return H3_ERR_NULL;
    if (n_mod_groups < 1) return H3_ERR_SHAPE;
    if (ld_mod_group < hidden && n_mod_groups > 1) return H3_ERR_SHAPE;
    if (ld_mod_group % 4 != 0) return H3_ERR_ALIGN;
    if (!aligned16(shift) || !aligned16(scale) || (gate && !aligned16(gate))) return H3_ERR_ALIGN;
    H3_TRY(check_bf16_mat(x, ld_x, hidden));
    H3_TRY(check_bf16_mat(h_out, ld_h, hidden));
    if (branch) {
        H3_TRY(check_bf16_mat(branch, ld_b, hidden));
        H3_TRY(check_bf16_mat(x1_out, ld_x1, hidden));
    }
    const Mat mx = mat(x, L_buf, hidden, ld_x), mh = mat(h_out, L_buf, hidden, ld_h);
    const Mat mb = mat(branch, branch ? L_buf : 0, hidden, ld_b);
    const Mat m1 = mat(x1_out, branch ? L_buf : 0, hidden, ld_x1);
    const int64_t modrows = n_mod_groups;
    const Mat msh = mat(shift, modrows, hidden, std::max<int64_t>(ld_mod_group, hidden), 4);
    const Mat msc = mat(scale, modrows, hidden, std::max<int64_t>(ld_mod_group, hidden), 4);
    const Mat mg = mat(gate, gate ? modrows : 0, hidden, std::max<int64_t>(ld_mod_group, hidden), 4);
    for (const Mat *in : {&mx, &mb, &msh, &msc, &mg})
        if (overlap(mh, *in)) return H3_ERR_ALIAS;
    if (branch) {
        if (overlap(m1, mh)) return H3_ERR_ALIAS;
        if (!same(m1, mx) && overlap(m1, mx)) return H3_ERR_ALIAS;
        for (const Mat *in : {&mb, &msh, &msc, &mg})
            if (overlap(m1, *in)) return H3_ERR_ALIAS;
    }
    return H3_OK;
}

int h3_check_qk_norm_rope(const uint16_t *q, const uint16_t *k, int64_t ld, const uint16_t *q_gain,
                          const uint16_t *k_gain, int64_t L_buf, int64_t valid_len, int32_t heads,
                          int32_t head_dim, int32_t rot_dim, int32_t pairing, float theta, float eps) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (heads <= 0 || head_dim <= 0) return H3_ERR_SHAPE;
    if (head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
    if ((int64_t)heads * head_dim > kMaxHidden) return H3_ERR_UNSUPPORTED;
    if (rot_dim < 0 || rot_dim > head_dim || rot_dim % 16 != 0) return H3_ERR_UNSUPPORTED;
    if (pairing != 0 && pairing != 1) return H3_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
    if (!(theta > 0.0f) || !std::isfinite(theta)) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    if (!q || !k || !q_gain || !k_gain) return H3_ERR_NULL;
    const int64_t H = (int64_t)heads * head_dim;
    H3_TRY(check_bf16_mat(q, ld, H));
    H3_TRY(check_bf16_mat(k, ld, H));
    if (!aligned16(q_gain) || !aligned16(k_gain)) return H3_ERR_ALIGN;
    const Mat mq = mat(q, L_buf, H, ld), mk = mat(k, L_buf, H, ld);
    if (overlap(mq, mk)) return H3_ERR_ALIAS;
    const Mat gq = mat(q_gain, 1, head_dim, head_dim), gk = mat(k_gain, 1, head_dim, head_dim);
    if (overlap(mq, gq) || overlap(mq, gk) || overlap(mk, gq) || overlap(mk, gk)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_swiglu(const uint16_t *u, int64_t ld_u, const uint16_t *g, int64_t ld_g, int64_t L_buf,
                    int64_t valid_len, int32_t ffn) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (ffn <= 0) return H3_ERR_SHAPE;
    if (ffn % 8 != 0) return H3_ERR_ALIGN;
    if (L_buf == 0) return H3_OK;
    if (!u || !g) return H3_ERR_NULL;
    H3_TRY(check_bf16_mat(u, ld_u, 2 * (int64_t)ffn));
    H3_TRY(check_bf16_mat(g, ld_g, ffn));
    if (overlap(mat(u, L_buf, 2 * (int64_t)ffn, ld_u), mat(g, L_buf, ffn, ld_g))) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_qk_norm_rope_lora(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t ld,
                               const uint16_t *dq, const uint16_t *dk, const uint16_t *dv, int64_t ld_d,
                               const uint16_t *q_gain, const uint16_t *k_gain, int64_t L_buf, int64_t valid_len,
                               int32_t heads, int32_t head_dim, int32_t rot_dim, int32_t pairing, float theta,
                               float eps) {
    H3_TRY(h3_check_qk_norm_rope(q, k, ld, q_gain, k_gain, L_buf, valid_len, heads, head_dim, rot_dim, pairing,
                                 theta, eps));
    if (L_buf == 0) return H3_OK;
    if (!dq || !dk || (v && !dv)) return H3_ERR_NULL;
    const int64_t H = (int64_t)heads * head_dim;
    H3_TRY(check_bf16_mat(dq, ld_d, H));
    H3_TRY(check_bf16_mat(dk, ld_d, H));
    const Mat mq = mat(q, L_buf, H, ld), mk = mat(k, L_buf, H, ld), mv = mat(v, v ? L_buf : 0, H, ld);
    if (v) {
        H3_TRY(check_bf16_mat(v, ld, H));
        H3_TRY(check_bf16_mat(dv, ld_d, H));
        if (overlap(mv, mq) || overlap(mv, mk)) return H3_ERR_ALIAS;
        const Mat gq = mat(q_gain, 1, head_dim, head_dim), gk = mat(k_gain, 1, head_dim, head_dim);
        if (overlap(mv, gq) || overlap(mv, gk)) return H3_ERR_ALIAS;
    }
    const Mat mdq = mat(dq, L_buf, H, ld_d), mdk = mat(dk, L_buf, H, ld_d), mdv = mat(dv, v ? L_buf : 0, H, ld_d);
    for (const Mat *out : {&mq, &mk, &mv})
        for (const Mat *d : {&mdq, &mdk, &mdv})
            if (overlap(*out, *d)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_fused_modulate_norm_lora(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                      const uint16_t *delta, int64_t ld_d, const float *shift, const float *scale,
                                      const float *gate, int64_t ld_mod_group, int32_t n_mod_groups,
                                      const uint16_t *x1_out, int64_t ld_x1, const uint16_t *h_out, int64_t ld_h,
                                      int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                      int32_t norm_type, int32_t gate_bf16) {
    (void)gate_bf16;
    H3_TRY(check_rows(L_buf, valid_len));
    if (L_buf > 0 && (!branch || !delta || !gate || !x1_out)) return H3_ERR_NULL;
    if (h_out) {
        H3_TRY(h3_check_fused_modulate_norm(x, ld_x, branch, ld_b, shift, scale, gate, ld_mod_group, n_mod_groups,
                                            x1_out, ld_x1, h_out, ld_h, L_buf, valid_len, hidden, eps, norm_type));
    } else {
        // residual only: the plain checks with the h output and the norm table
        // left out
        if (hidden <= 0) return H3_ERR_SHAPE;
        if (hidden > kMaxHidden) return H3_ERR_UNSUPPORTED;
        if (hidden % 8 != 0) return H3_ERR_ALIGN;
        if (norm_type != 0 && norm_type != 1) return H3_ERR_UNSUPPORTED;
        if (L_buf == 0) return H3_OK;
        if (!x) return H3_ERR_NULL;
        if (n_mod_groups < 1) return H3_ERR_SHAPE;
        if (ld_mod_group < hidden && n_mod_groups > 1) return H3_ERR_SHAPE;
        if (ld_mod_group % 4 != 0 || !aligned16(gate)) return H3_ERR_ALIGN;
        H3_TRY(check_bf16_mat(x, ld_x, hidden));
        H3_TRY(check_bf16_mat(branch, ld_b, hidden));
        H3_TRY(check_bf16_mat(x1_out, ld_x1, hidden));
        const Mat mx = mat(x, L_buf, hidden, ld_x), mb = mat(branch, L_buf, hidden, ld_b);
        const Mat m1 = mat(x1_out, L_buf, hidden, ld_x1);
        const Mat mg = mat(gate, n_mod_groups, hidden, std::max<int64_t>(ld_mod_group, hidden), 4);
        if (!same(m1, mx) && overlap(m1, mx)) return H3_ERR_ALIAS;
        if (overlap(m1, mb) || overlap(m1, mg)) return H3_ERR_ALIAS;
    }
    if (L_buf == 0) return H3_OK;
    H3_TRY(check_bf16_mat(delta, ld_d, hidden));
    const Mat md = mat(delta, L_buf, hidden, ld_d);
    if (overlap(mat(x1_out, L_buf, hidden, ld_x1), md)) return H3_ERR_ALIAS;
    if (h_out && overlap(mat(h_out, L_buf, hidden, ld_h), md)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_swiglu_lora(const uint16_t *u, int64_t ld_u, const uint16_t *du, int64_t ld_du, const uint16_t *g,
                         int64_t ld_g, int64_t L_buf, int64_t valid_len, int32_t ffn) {
    H3_TRY(h3_check_swiglu(u, ld_u, g, ld_g, L_buf, valid_len, ffn));
    if (L_buf == 0) return H3_OK;
    if (!du) return H3_ERR_NULL;
    H3_TRY(check_bf16_mat(du, ld_du, 2 * (int64_t)ffn));
    if (overlap(mat(du, L_buf, 2 * (int64_t)ffn, ld_du), mat(g, L_buf, ffn, ld_g))) return H3_ERR_ALIAS;
    return H3_OK;
}

size_t h3_linear_workspace_bytes(int64_t M_valid, int64_t N, int64_t K, int32_t epilogue) {
    if (M_valid < 0 || N <= 0 || K <= 0 || epilogue < H3_EPI_STORE || epilogue > H3_EPI_SWIGLU) return 0;
    return gemm_plan(M_valid, N, K, epilogue).ws_bytes;
}

int h3_check_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                    const uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                    int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                    int64_t ld_gate_group, int32_t n_mod_groups, const void *workspace, size_t ws_bytes) {
    H3_TRY(check_rows(M_buf, M_valid));
    if (N <= 0 || K <= 0) return H3_ERR_SHAPE;
    if (epilogue < H3_EPI_STORE || epilogue > H3_EPI_SWIGLU) return H3_ERR_UNSUPPORTED;
    if (N % 8 != 0 || K % 8 != 0) return H3_ERR_ALIGN;
    if (K % 64 != 0) return H3_ERR_UNSUPPORTED;  // the MFMA kernel steps K by 64
    if (epilogue == H3_EPI_SWIGLU && (N % 16) != 0) return H3_ERR_ALIGN;
    if (M_buf == 0) return H3_OK;
    if (!a || !w || !c) return H3_ERR_NULL;
    const int64_t Nc = epilogue == H3_EPI_SWIGLU ? N / 2 : N;
    H3_TRY(check_bf16_mat(a, lda, K));
    H3_TRY(check_bf16_mat(w, ldw, K));
    H3_TRY(check_bf16_mat(c, ldc, Nc));
    const Mat ma = mat(a, M_buf, K, lda), mw = mat(w, N, K, ldw), mc = mat(c, M_buf, Nc, ldc);
    if (overlap(mc, ma) || overlap(mc, mw)) return H3_ERR_ALIAS;
    if (bias) {
        if (!aligned16(bias)) return H3_ERR_ALIGN;
        if (overlap(mc, mat(bias, 1, N, N))) return H3_ERR_ALIAS;
    }
    if (epilogue == H3_EPI_RESIDUAL) {
        if (!resid || !gate) return H3_ERR_NULL;
        if (n_mod_groups < 1) return H3_ERR_SHAPE;
        if (!aligned16(gate)) return H3_ERR_ALIGN;
        // the gate table: n_mod_groups entries of N floats, ld_gate_group apart
        if (n_mod_groups > 1 && ld_gate_group < N) return H3_ERR_SHAPE;
        if (n_mod_groups > 1 && (ld_gate_group % 4) != 0) return H3_ERR_ALIGN;
        const Mat mg = mat(gate, n_mod_groups, N, n_mod_groups > 1 ? ld_gate_group : N, 4);
        if (overlap(mg, mc)) return H3_ERR_ALIAS;
        H3_TRY(check_bf16_mat(resid, ld_r, N));
        const Mat mr = mat(resid, M_buf, N, ld_r);
        if (!same(mr, mc) && overlap(mr, mc)) return H3_ERR_ALIAS;
    }
    if (workspace != nullptr) {
        const size_t need = gemm_plan(M_valid, N, K, epilogue).ws_bytes;
        if (ws_bytes < need) return H3_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return H3_ERR_ALIGN;
        if (need > 0) {
            const Mat mws = mat(workspace, 1, (int64_t)need, (int64_t)need, 1);
            if (overlap(mws, ma) || overlap(mws, mw) || overlap(mws, mc)) return H3_ERR_ALIAS;
            if (bias && overlap(mws, mat(bias, 1, N, N))) return H3_ERR_ALIAS;
            if (epilogue == H3_EPI_RESIDUAL &&
                (overlap(mws, mat(resid, M_buf, N, ld_r)) ||
                 overlap(mws, mat(gate, n_mod_groups, N, n_mod_groups > 1 ? ld_gate_group : N, 4))))
                return H3_ERR_ALIAS;
        }
    }
    return H3_OK;
}

// The staged V^T plane and key norms of an external segment (h3_kv_stage).
static int check_staged_seg(const h3_kv_seg &s, int64_t heads, std::vector<Mat> &planes) {
    if ((s.vt == nullptr) != (s.kmax2 == nullptr)) return H3_ERR_NULL;
    if (s.vt == nullptr) return H3_OK;
    if (s.k == nullptr) return H3_ERR_UNSUPPORTED;  // own rows are staged by the call itself
    if (!aligned16(s.vt) || (reinterpret_cast<uintptr_t>(s.kmax2) & 3u)) return H3_ERR_ALIGN;
    const int64_t bytes = heads * kHeadDim * ((s.len + 63) / 64 * 64) * 2;
    planes.push_back(mat(s.vt, 1, bytes, bytes, 1));
    planes.push_back(mat(s.kmax2, 1, heads, heads, 4));
    return H3_OK;
}

size_t h3_kv_stage_bytes(int64_t len, int32_t heads) {
    if (len < 0 || heads <= 0) return 0;
    return (size_t)heads * kHeadDim * ((len + 63) / 64 * 64) * 2;
}

int h3_check_mfma_ceiling(int32_t dtype, int32_t iters, const float *sink, int64_t sink_floats, const double *flops) {
    if (dtype != H3_CEIL_BF16 && dtype != H3_CEIL_FP8) return H3_ERR_UNSUPPORTED;
    if (!sink || !flops) return H3_ERR_NULL;
    if (iters < 1 || iters > (1 << 20) || sink_floats < 256) return H3_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return H3_ERR_ALIGN;
    return H3_OK;
}

int h3_check_kv_stage(const uint16_t *k, const uint16_t *v, int64_t ld, int64_t len, int32_t heads,
                      int32_t head_dim, const uint16_t *vt, const float *kmax2) {
    if (heads <= 0 || len < 0) return H3_ERR_SHAPE;
    if (head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
    if ((int64_t)heads * head_dim > kMaxHidden) return H3_ERR_SHAPE;
    if (len == 0) return H3_OK;
    if (!k || !v || !vt || !kmax2) return H3_ERR_NULL;
    const int64_t H = (int64_t)heads * head_dim;
    H3_TRY(check_bf16_mat(k, ld, H));
    H3_TRY(check_bf16_mat(v, ld, H));
    if (!aligned16(vt) || (reinterpret_cast<uintptr_t>(kmax2) & 3u)) return H3_ERR_ALIGN;
    const int64_t bytes = (int64_t)h3_kv_stage_bytes(len, heads);
    const Mat mvt = mat(vt, 1, bytes, bytes, 1), mk2 = mat(kmax2, 1, heads, heads, 4);
    const Mat mk = mat(k, len, H, ld), mv = mat(v, len, H, ld);
    if (overlap(mvt, mk) || overlap(mvt, mv) || overlap(mk2, mk) || overlap(mk2, mv) || overlap(mvt, mk2))
        return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                       const uint16_t *v, int64_t ld_v, const uint16_t *o, int64_t ld_o, int64_t L_buf,
                       int64_t valid_len, int32_t heads, int32_t head_dim, float softmax_scale,
                       const h3_qgroup *groups, int32_t n_groups, const void *workspace, size_t ws_bytes) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (heads <= 0 || head_dim <= 0) return H3_ERR_SHAPE;
    if (head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f) return H3_ERR_SHAPE;
    const int64_t H = (int64_t)heads * head_dim;
    if (groups != nullptr && (n_groups < 1 || n_groups > H3_MAX_GROUPS)) return H3_ERR_SHAPE;
    if (groups == nullptr && n_groups != 0) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    if (!q || !k || !v || !o) return H3_ERR_NULL;
    H3_TRY(check_bf16_mat(q, ld_q, H));
    H3_TRY(check_bf16_mat(k, ld_k, H));
    H3_TRY(check_bf16_mat(v, ld_v, H));
    H3_TRY(check_bf16_mat(o, ld_o, H));
    const Mat mo = mat(o, L_buf, H, ld_o);
    if (overlap(mo, mat(q, L_buf, H, ld_q)) || overlap(mo, mat(k, L_buf, H, ld_k)) ||
        overlap(mo, mat(v, L_buf, H, ld_v)))
        return H3_ERR_ALIAS;
    if (groups) {
        std::vector<std::pair<int64_t, int64_t>> spans;
        for (int gi = 0; gi < n_groups; ++gi) {
            const h3_qgroup &g = groups[gi];
            if (g.reserved != 0) return H3_ERR_SHAPE;
            if (g.q_begin < 0 || g.q_end < g.q_begin || g.q_end > valid_len) return H3_ERR_SHAPE;
            if (g.n_seg < 1 || g.n_seg > H3_MAX_SEGMENTS) return H3_ERR_UNSUPPORTED;
            if (g.q_end > g.q_begin) spans.push_back({g.q_begin, g.q_end});
            for (int si = 0; si < g.n_seg; ++si) {
                const h3_kv_seg &s = g.seg[si];
                if (s.begin < 0 || s.len < 1) return H3_ERR_SHAPE;
                if (s.k == nullptr) {
                    if (s.v != nullptr) return H3_ERR_NULL;
                    if (s.begin + s.len > valid_len) return H3_ERR_SHAPE;
                } else {
                    if (s.v == nullptr) return H3_ERR_NULL;
                    H3_TRY(check_bf16_mat(s.k, s.ld, H));
                    H3_TRY(check_bf16_mat(s.v, s.ld, H));
                    const Mat sk = mat(s.k + s.begin * s.ld, s.len, H, s.ld);
                    const Mat sv = mat(s.v + s.begin * s.ld, s.len, H, s.ld);
                    if (overlap(mo, sk) || overlap(mo, sv)) return H3_ERR_ALIAS;
                }
                std::vector<Mat> staged;
                H3_TRY(check_staged_seg(s, heads, staged));
                for (const Mat &m : staged) {
                    if (overlap(m, mo)) return H3_ERR_ALIAS;
                    if (workspace != nullptr && overlap(m, mat(workspace, 1, (int64_t)ws_bytes, (int64_t)ws_bytes, 1)))
                        return H3_ERR_ALIAS;
                }
            }
        }
        std::sort(spans.begin(), spans.end());
        for (size_t i = 1; i < spans.size(); ++i)
            if (spans[i].first < spans[i - 1].second) return H3_ERR_SHAPE;
    }
    // V^T staging workspace
    VtPlan plan;
    vt_plan(groups, n_groups, valid_len, heads, &plan);
    if (plan.bytes > 0) {
        if (workspace == nullptr || ws_bytes < plan.bytes) return H3_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return H3_ERR_ALIGN;
        const Mat mw = mat(workspace, 1, (int64_t)plan.bytes, (int64_t)plan.bytes, 1);
        if (overlap(mw, mo) || overlap(mw, mat(q, L_buf, H, ld_q)) || overlap(mw, mat(k, L_buf, H, ld_k)) ||
            overlap(mw, mat(v, L_buf, H, ld_v)))
            return H3_ERR_ALIAS;
        for (int i = 0; i < plan.n; ++i) {
            const VtSeg &e = plan.seg[i];
            if (!e.own && (overlap(mw, mat(e.v + e.begin * e.ld, e.len, H, e.ld)) ||
                           overlap(mw, mat(e.k + e.begin * e.ld, e.len, H, e.ld))))
                return H3_ERR_ALIAS;
        }
    }
    return H3_OK;
}

int h3_check_block_forward(const h3_dims *dims, const h3_block_weights *w, const uint16_t *x, uint16_t *y,
                           const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                           const int32_t *pos, int64_t L_buf, int64_t valid_len, const h3_qgroup *groups,
                           int32_t n_groups, const h3_kv_export *kv_export, const void *workspace,
                           size_t ws_bytes) {
    (void)mod_idx;
    (void)pos;
    H3_TRY(check_dims(dims));
    H3_TRY(check_rows(L_buf, valid_len));
    if (w == nullptr) return H3_ERR_NULL;
    if (groups != nullptr && (n_groups < 1 || n_groups > H3_MAX_GROUPS)) return H3_ERR_SHAPE;
    if (groups == nullptr && n_groups != 0) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    const int64_t H = dims->hidden, F = dims->ffn, d = dims->head_dim;
    if (!x || !y || !mod) return H3_ERR_NULL;
    if (!w->w_qkv || !w->q_gain || !w->k_gain || !w->w_o || !w->w_up || !w->w_down) return H3_ERR_NULL;
    if (n_mod_groups < 1) return H3_ERR_SHAPE;
    if (!aligned16(mod)) return H3_ERR_ALIGN;
    H3_TRY(check_bf16_mat(x, H, H));
    H3_TRY(check_bf16_mat(y, H, H));
    for (const uint16_t *p : {w->w_qkv, w->b_qkv, w->q_gain, w->k_gain, w->w_o, w->b_o, w->w_up, w->b_up,
                              w->w_down, w->b_down})
        if (p && !aligned16(p)) return H3_ERR_ALIGN;
    // workspace
    WsLayout l;
    if (!ws_layout(dims, L_buf, groups, n_groups, &l)) return H3_ERR_SHAPE;
    if (workspace == nullptr || ws_bytes < l.total) return H3_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return H3_ERR_ALIGN;
    const Mat mx = mat(x, L_buf, H, H), my = mat(y, L_buf, H, H);
    const Mat mws = mat(workspace, 1, (int64_t)l.total, (int64_t)l.total, 1);
    const Mat weights[] = {mat(w->w_qkv, 3 * H, H, H), mat(w->b_qkv, w->b_qkv ? 1 : 0, 3 * H, 3 * H),
                           mat(w->q_gain, 1, d, d),     mat(w->k_gain, 1, d, d),
                           mat(w->w_o, H, H, H),        mat(w->b_o, w->b_o ? 1 : 0, H, H),
                           mat(w->w_up, 2 * F, H, H),   mat(w->b_up, w->b_up ? 1 : 0, 2 * F, 2 * F),
                           mat(w->w_down, H, F, F),     mat(w->b_down, w->b_down ? 1 : 0, H, H)};
    const Mat mmod = mat(mod, 1, (int64_t)n_mod_groups * 6 * H, (int64_t)n_mod_groups * 6 * H, 4);
    if (!same(mx, my) && overlap(mx, my)) return H3_ERR_ALIAS;
    if (overlap(my, mws) || overlap(mx, mws) || overlap(my, mmod) || overlap(mws, mmod)) return H3_ERR_ALIAS;
    for (const Mat &m : weights)
        if (overlap(my, m) || overlap(mws, m)) return H3_ERR_ALIAS;
    if (groups) {
        // Same rules as h3_attention on the block's own q~/k~/v inside the workspace.
        std::vector<std::pair<int64_t, int64_t>> spans;
        for (int gi = 0; gi < n_groups; ++gi) {
            const h3_qgroup &g = groups[gi];
            if (g.reserved != 0) return H3_ERR_SHAPE;
            if (g.q_begin < 0 || g.q_end < g.q_begin || g.q_end > valid_len) return H3_ERR_SHAPE;
            if (g.n_seg < 1 || g.n_seg > H3_MAX_SEGMENTS) return H3_ERR_UNSUPPORTED;
            if (g.q_end > g.q_begin) spans.push_back({g.q_begin, g.q_end});
            for (int si = 0; si < g.n_seg; ++si) {
                const h3_kv_seg &s = g.seg[si];
                if (s.begin < 0 || s.len < 1) return H3_ERR_SHAPE;
                if (s.k == nullptr) {
                    if (s.v != nullptr) return H3_ERR_NULL;
                    if (s.begin + s.len > valid_len) return H3_ERR_SHAPE;
                } else {
                    if (s.v == nullptr) return H3_ERR_NULL;
                    H3_TRY(check_bf16_mat(s.k, s.ld, H));
                    H3_TRY(check_bf16_mat(s.v, s.ld, H));
                    const Mat sk = mat(s.k + s.begin * s.ld, s.len, H, s.ld);
                    const Mat sv = mat(s.v + s.begin * s.ld, s.len, H, s.ld);
                    if (overlap(my, sk) || overlap(my, sv) || overlap(mws, sk) || overlap(mws, sv))
                        return H3_ERR_ALIAS;
                }
                std::vector<Mat> staged;
                H3_TRY(check_staged_seg(s, dims->heads, staged));
                for (const Mat &m : staged)
                    if (overlap(m, my) || overlap(m, mws)) return H3_ERR_ALIAS;
            }
        }
        std::sort(spans.begin(), spans.end());
        for (size_t i = 1; i < spans.size(); ++i)
            if (spans[i].first < spans[i - 1].second) return H3_ERR_SHAPE;
    }
    if (kv_export) {
        const h3_kv_export &e = *kv_export;
        if (!e.k || !e.v) return H3_ERR_NULL;
        if (e.src_begin < 0 || e.len < 0 || e.src_begin + e.len > valid_len) return H3_ERR_SHAPE;
        H3_TRY(check_bf16_mat(e.k, e.ld, H));
        H3_TRY(check_bf16_mat(e.v, e.ld, H));
        const Mat ek = mat(e.k, e.len, H, e.ld), ev = mat(e.v, e.len, H, e.ld);
        if (overlap(ek, ev)) return H3_ERR_ALIAS;
        for (const Mat *m : {&mx, &my, &mws, &mmod})
            if (overlap(ek, *m) || overlap(ev, *m)) return H3_ERR_ALIAS;
        for (const Mat &m : weights)
            if (overlap(ek, m) || overlap(ev, m)) return H3_ERR_ALIAS;
    }
    return H3_OK;
}


int h3_check_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, int64_t valid_len,
                           int64_t prefix_len, int32_t heads, int32_t head_dim, float tau, const uint16_t *blocks,
                           const int32_t *counts, const void *workspace, size_t ws_bytes) {
    if (valid_len < 0 || prefix_len < 0 || prefix_len > valid_len) return H3_ERR_SHAPE;
    if (heads <= 0 || head_dim <= 0) return H3_ERR_SHAPE;
    if (head_dim != kHeadDim) return H3_ERR_UNSUPPORTED;
    if (!std::isfinite(tau)) return H3_ERR_SHAPE;
    const int64_t T = valid_len - prefix_len;
    if (T > (int64_t)H3_SPARSE_MAX_KBLOCKS * H3_SPARSE_K_BLOCK) return H3_ERR_UNSUPPORTED;
    if (T == 0) return H3_OK;
    if (!q || !k || !blocks || !counts) return H3_ERR_NULL;
    const int64_t H = (int64_t)heads * head_dim;
    H3_TRY(check_bf16_mat(q, ld_q, H));
    H3_TRY(check_bf16_mat(k, ld_k, H));
    if ((reinterpret_cast<uintptr_t>(blocks) & 1u) || (reinterpret_cast<uintptr_t>(counts) & 3u)) return H3_ERR_ALIGN;
    SparseGeom g;
    sparse_geometry(valid_len, prefix_len, heads, &g);
    if (workspace == nullptr || ws_bytes < g.ws_bytes) return H3_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return H3_ERR_ALIGN;
    const Mat outs[3] = {bytes_of(blocks, (int64_t)heads * g.n_qb * g.n_kb * 2),
                         bytes_of(counts, (int64_t)heads * g.n_qb * 4), bytes_of(workspace, (int64_t)g.ws_bytes)};
    const Mat mq = mat(q, valid_len, H, ld_q), mk = mat(k, valid_len, H, ld_k);
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], mq) || overlap(outs[i], mk)) return H3_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return H3_ERR_ALIAS;
    }
    return H3_OK;
}

int h3_check_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                              int64_t ld_v, const uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len,
                              int64_t prefix_len, int32_t heads, int32_t head_dim, float softmax_scale,
                              const uint16_t *blocks, const int32_t *counts, const void *workspace,
                              size_t ws_bytes) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (prefix_len < 0 || prefix_len > valid_len) return H3_ERR_SHAPE;
    const int64_t T = valid_len - prefix_len;
    if (T > 0 && prefix_len < 1) return H3_ERR_SHAPE;  // target rows always attend to the prefix
    if (T > (int64_t)H3_SPARSE_MAX_KBLOCKS * H3_SPARSE_K_BLOCK) return H3_ERR_UNSUPPORTED;
    if (T == 0)
        return h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim,
                                  softmax_scale, nullptr, 0, workspace, ws_bytes);
    h3_qgroup g;
    sparse_vt_group(valid_len, prefix_len, &g);
    H3_TRY(h3_check_attention(q, ld_q, k, ld_k, v, ld_v, o, ld_o, L_buf, valid_len, heads, head_dim, softmax_scale,
                              &g, 1, workspace, ws_bytes));
    if (!blocks || !counts) return H3_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(blocks) & 1u) || (reinterpret_cast<uintptr_t>(counts) & 3u)) return H3_ERR_ALIGN;
    SparseGeom sg;
    sparse_geometry(valid_len, prefix_len, heads, &sg);
    const int64_t H = (int64_t)heads * head_dim;
    const Mat mo = mat(o, L_buf, H, ld_o);
    const Mat mb = bytes_of(blocks, (int64_t)heads * sg.n_qb * sg.n_kb * 2);
    const Mat mc = bytes_of(counts, (int64_t)heads * sg.n_qb * 4);
    const Mat mw = bytes_of(workspace, (int64_t)h3_sparse_attention_workspace_bytes(valid_len, prefix_len, heads));
    if (overlap(mo, mb) || overlap(mo, mc) || overlap(mw, mb) || overlap(mw, mc)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_stack_forward(const h3_dims *dims, const h3_block_weights *w, int32_t n_blocks, const uint16_t *x,
                           const float *mod, int64_t ld_mod_block, int32_t n_mod_groups, const int32_t *mod_idx,
                           const int32_t *pos, int64_t L_buf, int64_t valid_len, const void *workspace,
                           size_t ws_bytes) {
    H3_TRY(check_dims(dims));
    H3_TRY(check_rows(L_buf, valid_len));
    if (n_blocks < 0 || ld_mod_block < 0 || ld_mod_block > (int64_t(1) << 40)) return H3_ERR_SHAPE;
    if (ld_mod_block % 4 != 0) return H3_ERR_ALIGN;
    if (n_blocks == 0) return H3_OK;
    if (w == nullptr || mod == nullptr) return H3_ERR_NULL;
    uint16_t *xm = const_cast<uint16_t *>(x);  // the stack writes x in place
    for (int32_t b = 0; b < n_blocks; ++b)
        H3_TRY(h3_check_block_forward(dims, w + b, x, xm, mod + (int64_t)b * ld_mod_block, n_mod_groups, mod_idx,
                                      pos, L_buf, valid_len, nullptr, 0, nullptr, workspace, ws_bytes));
    return H3_OK;
}

int h3_check_block_forward_sparse(const h3_dims *dims, const h3_block_weights *w, const uint16_t *x, uint16_t *y,
                                  const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                  const int32_t *pos, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                  float tau, const void *workspace, size_t ws_bytes) {
    H3_TRY(h3_check_block_forward(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len, nullptr, 0,
                                  nullptr, workspace, ws_bytes));
    if (prefix_len < 0 || prefix_len > valid_len) return H3_ERR_SHAPE;
    const int64_t T = valid_len - prefix_len;
    if (T > 0 && prefix_len < 1) return H3_ERR_SHAPE;
    if (T > (int64_t)H3_SPARSE_MAX_KBLOCKS * H3_SPARSE_K_BLOCK) return H3_ERR_UNSUPPORTED;
    if (!std::isfinite(tau)) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    BlockSparseLayout l;
    if (!block_sparse_layout(dims, L_buf, valid_len, prefix_len, &l)) return H3_ERR_SHAPE;
    if (ws_bytes < l.total) return H3_ERR_WORKSPACE;
    // The dense block's check covered the workspace's first dense-layout bytes;
    // the rest must not overlap the inputs, the output or the weights either.
    WsLayout dl;
    ws_layout(dims, L_buf, nullptr, 0, &dl);
    const int64_t H = dims->hidden, F = dims->ffn, d = dims->head_dim;
    const Mat extra = bytes_of(static_cast<const uint8_t *>(workspace) + dl.total, (int64_t)(l.total - dl.total));
    const Mat others[] = {mat(x, L_buf, H, H),
                          mat(y, L_buf, H, H),
                          mat(mod, 1, (int64_t)n_mod_groups * 6 * H, (int64_t)n_mod_groups * 6 * H, 4),
                          mat(w->w_qkv, 3 * H, H, H),
                          mat(w->b_qkv, w->b_qkv ? 1 : 0, 3 * H, 3 * H),
                          mat(w->q_gain, 1, d, d),
                          mat(w->k_gain, 1, d, d),
                          mat(w->w_o, H, H, H),
                          mat(w->b_o, w->b_o ? 1 : 0, H, H),
                          mat(w->w_up, 2 * F, H, H),
                          mat(w->b_up, w->b_up ? 1 : 0, 2 * F, 2 * F),
                          mat(w->w_down, H, F, F),
                          mat(w->b_down, w->b_down ? 1 : 0, H, H)};
    for (const Mat &m : others)
        if (overlap(extra, m)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_mxfp8_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K,
                            const uint8_t *q, int64_t ld_q, const uint8_t *scales) {
    H3_TRY(check_rows(rows_buf, rows_valid));
    if (K <= 0) return H3_ERR_SHAPE;
    if (K % 128 != 0) return H3_ERR_UNSUPPORTED;  // scales are stored per 128-wide slab
    if (rows_buf == 0) return H3_OK;
    if (!q || !scales || (rows_valid > 0 && !x)) return H3_ERR_NULL;
    if (rows_valid > 0) H3_TRY(check_bf16_mat(x, ld_x, K));
    if (ld_q < K) return H3_ERR_SHAPE;
    if (!aligned16(q) || (ld_q % 16) != 0 || (reinterpret_cast<uintptr_t>(scales) & 3u)) return H3_ERR_ALIGN;
    const Mat mx = mat(x, rows_valid, K, ld_x), mq = mat(q, rows_buf, K, ld_q, 1);
    const Mat ms = bytes_of(scales, rows_buf * (K / 32));
    if (overlap(mq, mx) || overlap(ms, mx) || overlap(ms, mq)) return H3_ERR_ALIAS;
    return H3_OK;
}

int h3_check_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                          const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias,
                          const uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                          int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                          int64_t ld_gate_group, int32_t n_mod_groups) {
    H3_TRY(check_rows(M_buf, M_valid));
    if (N <= 0 || K <= 0) return H3_ERR_SHAPE;
    if (epilogue < H3_EPI_STORE || epilogue > H3_EPI_SWIGLU) return H3_ERR_UNSUPPORTED;
    if (N % 8 != 0) return H3_ERR_ALIGN;
    if (K % 128 != 0) return H3_ERR_UNSUPPORTED;  // the kernel's K stage and the scale slabs
    if (epilogue == H3_EPI_SWIGLU && (N % 16) != 0) return H3_ERR_ALIGN;
    if (M_buf == 0) return H3_OK;
    if (!a || !w || !c || !a_scales || !w_scales) return H3_ERR_NULL;
    if (a_scale_rows < M_valid) return H3_ERR_SHAPE;
    if (lda < K || ldw < K) return H3_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(w) || (lda % 16) != 0 || (ldw % 16) != 0) return H3_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scales) & 3u))
        return H3_ERR_ALIGN;
    if (bias && !aligned16(bias)) return H3_ERR_ALIGN;
    const int64_t Nc = epilogue == H3_EPI_SWIGLU ? N / 2 : N;
    H3_TRY(check_bf16_mat(c, ldc, Nc));
    const Mat ma = mat(a, M_buf, K, lda, 1), mw = mat(w, N, K, ldw, 1), mc = mat(c, M_buf, Nc, ldc);
    const Mat mas = bytes_of(a_scales, a_scale_rows * (K / 32)), mws = bytes_of(w_scales, N * (K / 32));
    if (overlap(mc, ma) || overlap(mc, mw) || overlap(mc, mas) || overlap(mc, mws)) return H3_ERR_ALIAS;
    if (epilogue == H3_EPI_RESIDUAL) {
        if (!resid || !gate) return H3_ERR_NULL;
        if (n_mod_groups < 1) return H3_ERR_SHAPE;
        if (!aligned16(gate)) return H3_ERR_ALIGN;
        if (n_mod_groups > 1 && ld_gate_group < N) return H3_ERR_SHAPE;
        if (n_mod_groups > 1 && (ld_gate_group % 4) != 0) return H3_ERR_ALIGN;
        if (overlap(mat(gate, n_mod_groups, N, n_mod_groups > 1 ? ld_gate_group : N, 4), mc)) return H3_ERR_ALIAS;
        H3_TRY(check_bf16_mat(resid, ld_r, N));
        const Mat mr = mat(resid, M_buf, N, ld_r);
        if (!same(mr, mc) && overlap(mr, mc)) return H3_ERR_ALIAS;
    }
    return H3_OK;
}

int h3_check_fused_modulate_norm_mxfp8(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                       const float *shift, const float *scale, const float *gate,
                                       int64_t ld_mod_group, int32_t n_mod_groups, const uint16_t *x1_out,
                                       int64_t ld_x1, const uint8_t *hq, int64_t ld_hq, const uint8_t *hs,
                                       int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                       int32_t norm_type) {
    H3_TRY(check_rows(L_buf, valid_len));
    if (hidden <= 0) return H3_ERR_SHAPE;
    if (hidden > kMaxHidden) return H3_ERR_UNSUPPORTED;
    if (hidden % 128 != 0) return H3_ERR_UNSUPPORTED;  // whole 128-wide scale slabs
    if (norm_type != 0 && norm_type != 1) return H3_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return H3_ERR_SHAPE;
    if (L_buf == 0) return H3_OK;
    if (!x || !hq || !hs || !shift || !scale) return H3_ERR_NULL;
    if (branch && (!gate || !x1_out)) return H3_ERR_NULL;
    if (n_mod_groups < 1) return H3_ERR_SHAPE;
    if (ld_mod_group < hidden && n_mod_groups > 1) return H3_ERR_SHAPE;
    if (ld_mod_group % 4 != 0) return H3_ERR_ALIGN;
    if (!aligned16(shift) || !aligned16(scale) || (gate && !aligned16(gate))) return H3_ERR_ALIGN;
    H3_TRY(check_bf16_mat(x, ld_x, hidden));
    if (ld_hq < hidden) return H3_ERR_SHAPE;
    if (!aligned16(hq) || (ld_hq % 16) != 0 || (reinterpret_cast<uintptr_t>(hs) & 3u)) return H3_ERR_ALIGN;
    if (branch) {
        H3_TRY(check_bf16_mat(branch, ld_b, hidden));
        H3_TRY(check_bf16_mat(x1_out, ld_x1, hidden));
    }
    const Mat mx = mat(x, L_buf, hidden, ld_x), mq = mat(hq, L_buf, hidden, ld_hq, 1);
    const Mat ms = bytes_of(hs, L_buf * (hidden / 32));
    const Mat mb = mat(branch, branch ? L_buf : 0, hidden, ld_b);
    const Mat m1 = mat(x1_out, branch ? L_buf : 0, hidden, ld_x1);
    const int64_t lm = std::max<int64_t>(ld_mod_group, hidden);
    const Mat msh = mat(shift, n_mod_groups, hidden, lm, 4), msc = mat(scale, n_mod_groups, hidden, lm, 4);
    const Mat mg = mat(gate, gate ? n_mod_groups : 0, hidden, lm, 4);
    for (const Mat *out : {&mq, &ms})
        for (const Mat *in : {&mx, &mb, &msh, &msc, &mg, &m1})
            if (overlap(*out, *in)) return H3_ERR_ALIAS;
    if (overlap(mq, ms)) return H3_ERR_ALIAS;
    if (branch) {
        if (!same(m1, mx) && overlap(m1, mx)) return H3_ERR_ALIAS;
        for (const Mat *in : {&mb, &msh, &msc, &mg})
            if (overlap(m1, *in)) return H3_ERR_ALIAS;
    }
    return H3_OK;
}

size_t h3_block_mxfp8_workspace_bytes(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len) {
    MxWsLayout l;
    if (!mx_ws_layout(dims, L_buf, valid_len, prefix_len, &l)) return 0;
    return l.total;
}

int h3_block_mxfp8_workspace_layout(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                    int64_t offsets[H3_MXWS_COUNT]) {
    if (offsets == nullptr) return H3_ERR_NULL;
    H3_TRY(check_dims(dims));
    if (L_buf < 0 || valid_len < 0 || valid_len > L_buf) return H3_ERR_SHAPE;
    MxWsLayout l;
    if (!mx_ws_layout(dims, L_buf, valid_len, prefix_len, &l)) return H3_ERR_UNSUPPORTED;
    for (int i = 0; i < H3_MXWS_COUNT; ++i) offsets[i] = l.off[i];
    return H3_OK;
}

int h3_check_block_forward_mxfp8(const h3_dims *dims, const h3_block_weights_mxfp8 *w, const uint16_t *x,
                                 const uint16_t *y, const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                 const int32_t *pos, int64_t L_buf, int64_t valid_len, int64_t prefix_len, float tau,
                                 const void *workspace, size_t ws_bytes) {
    (void)mod_idx;
    (void)pos;
    H3_TRY(check_dims(dims));
    if (dims->hidden % 128 != 0 || dims->ffn % 128 != 0) return H3_ERR_UNSUPPORTED;
    H3_TRY(check_rows(L_buf, valid_len));
    if (prefix_len >= 0) {
        if (prefix_len > valid_len) return H3_ERR_SHAPE;
        const int64_t T = valid_len - prefix_len;
        if (T > 0 && prefix_len < 1) return H3_ERR_SHAPE;
        if (T > (int64_t)H3_SPARSE_MAX_KBLOCKS * H3_SPARSE_K_BLOCK) return H3_ERR_UNSUPPORTED;
        if (!std::isfinite(tau)) return H3_ERR_SHAPE;
    }
    if (w == nullptr) return H3_ERR_NULL;
    if (L_buf == 0) return H3_OK;
    const int64_t H = dims->hidden, F = dims->ffn, d = dims->head_dim;
    if (!x || !y || !mod) return H3_ERR_NULL;
    if (!w->w_qkv || !w->s_qkv || !w->w_o || !w->s_o || !w->w_up || !w->s_up || !w->w_down || !w->s_down ||
        !w->q_gain || !w->k_gain)
        return H3_ERR_NULL;
    if (n_mod_groups < 1) return H3_ERR_SHAPE;
    if (!aligned16(mod)) return H3_ERR_ALIGN;
    H3_TRY(check_bf16_mat(x, H, H));
    H3_TRY(check_bf16_mat(y, H, H));
    for (const uint8_t *p : {w->w_qkv, w->w_o, w->w_up, w->w_down})
        if (!aligned16(p)) return H3_ERR_ALIGN;
    for (const uint8_t *p : {w->s_qkv, w->s_o, w->s_up, w->s_down})
        if (reinterpret_cast<uintptr_t>(p) & 3u) return H3_ERR_ALIGN;
    for (const uint16_t *p : {w->b_qkv, w->b_o, w->b_up, w->b_down, w->q_gain, w->k_gain})
        if (p && !aligned16(p)) return H3_ERR_ALIGN;
    MxWsLayout l;
    if (!mx_ws_layout(dims, L_buf, valid_len, prefix_len, &l)) return H3_ERR_SHAPE;
    if (workspace == nullptr || ws_bytes < l.total) return H3_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % kWsAlign) != 0) return H3_ERR_ALIGN;
    const Mat mx = mat(x, L_buf, H, H), my = mat(y, L_buf, H, H);
    const Mat mws = bytes_of(workspace, (int64_t)l.total);
    const Mat mmod = mat(mod, 1, (int64_t)n_mod_groups * 6 * H, (int64_t)n_mod_groups * 6 * H, 4);
    const Mat weights[] = {mat(w->w_qkv, 3 * H, H, H, 1), bytes_of(w->s_qkv, 3 * H * H / 32),
                           mat(w->w_o, H, H, H, 1),       bytes_of(w->s_o, H * H / 32),
                           mat(w->w_up, 2 * F, H, H, 1),  bytes_of(w->s_up, 2 * F * H / 32),
                           mat(w->w_down, H, F, F, 1),    bytes_of(w->s_down, H * F / 32),
                           mat(w->b_qkv, w->b_qkv ? 1 : 0, 3 * H, 3 * H), mat(w->b_o, w->b_o ? 1 : 0, H, H),
                           mat(w->b_up, w->b_up ? 1 : 0, 2 * F, 2 * F),   mat(w->b_down, w->b_down ? 1 : 0, H, H),
                           mat(w->q_gain, 1, d, d),       mat(w->k_gain, 1, d, d)};
    if (!same(mx, my) && overlap(mx, my)) return H3_ERR_ALIAS;
    if (overlap(my, mws) || overlap(mx, mws) || overlap(my, mmod) || overlap(mws, mmod)) return H3_ERR_ALIAS;
    for (const Mat &m : weights)
        if (overlap(my, m) || overlap(mws, m)) return H3_ERR_ALIAS;
    return H3_OK;
}

}  // extern "C"
