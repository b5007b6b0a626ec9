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
struct VtPlan {
    int n;
    VtSeg seg[H3_MAX_GROUPS * H3_MAX_SEGMENTS];
    int map[H3_MAX_GROUPS][H3_MAX_SEGMENTS];  // (group, segment) -> seg index
    int64_t kmax_off;     // byte offset of the per-head key norm maxima
    int64_t flags_off;    // byte offset of one int32 per attention workgroup
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
