// Internal declarations shared by the host-side sources of libh3block.
// Nothing here is part of the public ABI (include/h3block.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "h3block.h"

namespace h3 {

constexpr int64_t kHeadDim = 128;
constexpr int64_t kMaxHidden = 16384;
constexpr size_t kWsAlign = 256;

// Attention stages each distinct K/V segment's V transposed per head in the
// workspace: [heads][128][lpad] BF16 with lpad = len rounded up to 64.
// Segments are identified by (own rows or external pointer, stride, begin, len).
// After the segments come one FP32 per head, the largest squared norm of the
// call's keys (it bounds every score), and one int32 per attention
// workgroup, which tells the online kernel instance which workgroups the
// fixed-reference instance left to it (see the attention kernel).
struct VtSeg {
    int own;              // rows of the call's own K/V
    const uint16_t *k;    // external K (own == 0)
    const uint16_t *v;    // external V (own == 0)
    int64_t ld, begin, len, lpad;
    int64_t off;          // byte offset inside the V^T staging area
};
// Work schedule of one attention launch. A work item is one 256-row query
// tile of one head of one group ("(head, tile) item"), or a piece of one: its
// keys cut into `split` consecutive ranges of key tiles whose partial
// results a merge pass combines. Ranges of items are dispatched in order:
// the group whose items read the most keys first; if it fills less than
// four rounds of the chip's 256 workgroup slots, its last, partial round is
// cut into pieces (2 to 4, at least 4 key tiles each: the count whose tail,
// with the other groups' items after it, finishes soonest under list
// scheduling, if any beats 1);
// then the other groups, longest items first. With more than one range, each
// range is padded to a multiple of 8 items so that it starts on XCD 0 (also
// a single range cut into pieces).
constexpr int kAttnSlots = 256;
// int32 words of an attention launch's work queue (ticket counters).
constexpr int kAttnQueueWords = 16;
// Fixed cost of one work item (Q loads, the first tiles' latency, the
// epilogue), in key tiles of the steady loop: about 15 us against 1.8 us per
// tile, measured on full rounds of short items.
constexpr int64_t kAttnItemTiles = 8;
// At most this many of the other groups' items enter the tail's estimate.
constexpr int64_t kAttnSimUnits = 2048;
struct AttnSchedule {
    int n;                                // ranges
    int group[H3_MAX_GROUPS + 1];         // caller's group index of each range
    int32_t first[H3_MAX_GROUPS + 1];     // first (head, tile) item of the group in the range
    int32_t count[H3_MAX_GROUPS + 1];     // (head, tile) items in the range
    int32_t split[H3_MAX_GROUPS + 1];     // pieces per item (1: whole)
    int32_t end[H3_MAX_GROUPS + 1];       // exclusive end of the range's work items
    int32_t items;                        // work items of the launch
    int32_t split_items, pieces;          // (head, tile) items cut into pieces, pieces per item
};
// groups == NULL schedules one dense group of dense_len rows over keys [0, dense_len).
void attn_schedule(const h3_qgroup *groups, int n_groups, int64_t dense_len, int heads, AttnSchedule *out);

struct VtPlan {
    int n;
    VtSeg seg[H3_MAX_GROUPS * H3_MAX_SEGMENTS];
    int map[H3_MAX_GROUPS][H3_MAX_SEGMENTS];  // (group, segment) -> seg index
    int64_t part_off;     // byte offset of the split items' partial results (FP32 O, then (m, l) per row)
    int64_t kmax_off;     // byte offset of the per-head key norm maxima
    int64_t flags_off;    // byte offset of one int32 per attention work item (the deferred-item list)
    int64_t queue_off;    // byte offset of the launch's kAttnQueueWords work-queue words
    size_t bytes;
};
// groups == NULL plans one own segment [0, dense_len).
void vt_plan(const h3_qgroup *groups, int n_groups, int64_t dense_len, int heads, VtPlan *out);

// Geometry of Sol-Attn block selection over target rows [P, valid_len):
// query blocks of H3_SPARSE_Q_BLOCK rows, KV blocks of H3_SPARSE_K_BLOCK rows,
// and the selection workspace (FP32 query-block means [heads][n_qb][128], then
// transposed KV-block means [heads][128][n_kb_pad]).
struct SparseGeom {
    int64_t T;                 // target rows
    int64_t n_qb, n_kb;        // query / KV blocks
    int64_t per, n_kb_pad;     // KV blocks per selection thread (multiple of 4); 256 * per
    int64_t qbar_off, kbar_off;
    size_t ws_bytes;
};
void sparse_geometry(int64_t valid_len, int64_t prefix_len, int32_t heads, SparseGeom *g);
// The block-sparse attention's two key segments as one query group over
// [0, valid_len): own rows [0, P) and [P, valid_len). Used to plan and check
// the V^T staging.
void sparse_vt_group(int64_t valid_len, int64_t prefix_len, h3_qgroup *g);

// Launch plan of one BF16 GEMM (h3_linear): 256 x 256 output tiles in the
// grouped order, K in stages of 64. When the last round of tiles fills at
// most 4/5 of the chip's 256 workgroup slots and leaves the equivalent of at
// least kSkWorthStages stages idle (stages x idle share), that tail
// (sk_tiles tiles) is
// cut into sk_groups equal ranges of (tile, stage) units, at least
// kSkMinStages stages each and less than one tile (so a range touches at
// most two tiles), whose FP32 partial sums a fix-up pass adds; the other
// dp_tiles tiles run one per workgroup. sk_groups == 0: no tail split.
//
// Tile dealing: when the dp_tiles fill at least kGemmDealRounds rounds, the
// last W = max(96, T/12) of each XCD's T tiles are drawn by workgroups from
// a per-XCD counter (W + W/2 drawing workgroups per XCD; grid workgroups in
// all), which lets faster XCDs take over the end of slower ones' ranges. The
// counters sit at queue_off in the workspace (256 bytes).
constexpr int kGemmSlots = 256;
constexpr int kSkMinStages = 8;
constexpr int kSkWorthStages = 55;
constexpr int kGemmDealRounds = 8;
struct GemmPlan {
    int32_t tiles_m, tiles_n, tiles, stages;
    int32_t dp_tiles, sk_tiles, sk_groups;
    size_t part_bytes;  // 2 slots of 256 x 256 FP32 per range
    bool deal;          // tiles drawn from counters at the end of each XCD's range
    int32_t static_tickets, grid;
    size_t queue_off;
    size_t ws_bytes;    // workspace the plan needs (partial sums, then the counters)
};
GemmPlan gemm_plan(int64_t M_valid, int64_t N, int64_t K, int32_t epilogue);
// Largest ws_bytes of any plan with at most M_buf rows, for these (N, K, epilogue).
size_t gemm_ws_bytes_max(int64_t M_buf, int64_t N, int64_t K, int32_t epilogue);

// Byte offsets and row strides of the block's workspace buffers.
struct WsLayout {
    int64_t off[H3_WS_COUNT];
    int64_t ld[H3_WS_COUNT];
    int64_t cols[H3_WS_COUNT];
    size_t total;
};
bool ws_layout(const h3_dims *d, int64_t L_buf, const h3_qgroup *groups, int n_groups, WsLayout *out);

// Workspace of the block with block-sparse attention: the dense block's
// layout (the V^T slot grown to fit the two key segments if needed), then the
// selection lists, their counts and the selection's own workspace.
struct BlockSparseLayout {
    WsLayout base;
    int64_t blocks_off, counts_off, select_off;
    size_t total;
};
bool block_sparse_layout(const h3_dims *d, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                         BlockSparseLayout *out);

// Workspace of the MXFP8 block: byte offsets of the H3_MXWS_* buffers.
struct MxWsLayout {
    int64_t off[H3_MXWS_COUNT];
    size_t total;
};
// prefix_len < 0 (or >= valid_len): dense attention, the selection entries
// are empty.
bool mx_ws_layout(const h3_dims *d, int64_t L_buf, int64_t valid_len, int64_t prefix_len, MxWsLayout *out);

// Validation of dims shared by several checks.
int check_dims(const h3_dims *d);

}  // namespace h3
