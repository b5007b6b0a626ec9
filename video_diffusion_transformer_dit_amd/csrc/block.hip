// h3_block_forward: one MiniMax-H3 DiT block over a packed token sequence,
// composed from the library's kernels on the caller's stream (Sol-H3 report,
// §3.5 "Kernel Fusion": the three operator groups around the projections;
// vLLM-Omni H3 blog, §3.1-3.2).
//
//   1 modnorm        h   = RMSNorm(x) (1 + scale_a) + shift_a           group (1)
//   2 GEMM           qkv = h W_qkv^T (+ b)                               packed QKV
//   3 qk-norm+RoPE   q~, k~ in place in qkv                              group (2)
//   4 attention      o   = softmax(q~ k~^T / sqrt(128)) v
//   5 GEMM+residual  x1  = x + gate_a (o W_o^T (+ b))                    group (1)
//   6 modnorm        h2  = RMSNorm(x1) (1 + scale_f) + shift_f           group (1)
//   7 GEMM+SwiGLU    g   = silu(h2 W_gate^T) * (h2 W_up^T)               group (3)
//   8 GEMM+residual  y   = x1 + gate_f (g W_down^T (+ b))                group (1)
//   9 KV export      (refresh forwards only) copy k~ and v rows out
// Every kernel works on the valid rows only; padding rows of every output and
// intermediate are written as zero. The block-sparse variant replaces step 4
// by the Sol-Attn block selection and the list-mode attention (Sol-H3 report,
// §3.4 "Sparse Attention").
#include "h3_gemm_epilogue.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

struct SparseStep {
    int64_t prefix_len;
    float tau;
    const BlockSparseLayout *l;
};

// Steps 1-9 on the caller's stream; arguments already validated.
void block_steps(const h3_dims *dims, const h3_block_weights *w, const uint16_t *x, uint16_t *y, const float *mod,
                 int32_t n_mod_groups, const int32_t *mod_idx, const int32_t *pos, int64_t L_buf,
                 int64_t valid_len, const h3_qgroup *groups, int32_t n_groups, const h3_kv_export *kv_export,
                 const WsLayout &l, void *workspace, const SparseStep *sp, hipStream_t st) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_H]);
    uint16_t *qkv = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_QKV]);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_O]);
    uint16_t *x1 = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_X1]);
    uint16_t *h2 = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_H2]);
    uint16_t *g = reinterpret_cast<uint16_t *>(ws + l.off[H3_WS_G]);
    void *vt = ws + l.off[H3_WS_VT];
    void *part = ws + l.off[H3_WS_GEMM];  // the projections' stream-K partial sums

    const int64_t H = dims->hidden, F = dims->ffn, V = valid_len;
    const int64_t ldm = 6 * H;  // floats between modulation-table entries
    const float *shift_a = mod, *scale_a = mod + H, *gate_a = mod + 2 * H;
    const float *shift_f = mod + 3 * H, *scale_f = mod + 4 * H, *gate_f = mod + 5 * H;

    // 1 h
    launch_modnorm(x, H, nullptr, 0, shift_a, scale_a, nullptr, ldm, n_mod_groups, mod_idx, nullptr, 0, h, H, L_buf,
                   V, (int32_t)H, dims->eps, dims->norm_type, st);
    // 2 qkv
    launch_linear(h, H, w->w_qkv, H, w->b_qkv, qkv, 3 * H, V, 3 * H, H, H3_EPI_STORE, nullptr, 0, nullptr, 0, 1,
                  nullptr, st, part);
    launch_zero_rows(qkv, 3 * H, 3 * H, V, L_buf, st);
    // 3 q~, k~ (also zeroes their padding rows)
    launch_qk_norm_rope(qkv, qkv + H, 3 * H, w->q_gain, w->k_gain, pos, L_buf, V, dims->heads, dims->rot_dim,
                        dims->rope_pairing, dims->rope_theta, dims->eps, st);
    // 4 o
    if (sp == nullptr) {
        launch_attention(qkv, 3 * H, qkv + H, 3 * H, qkv + 2 * H, 3 * H, o, H, L_buf, V, dims->heads, 0.0f, groups,
                         n_groups, vt, st);
    } else {
        uint16_t *blocks = reinterpret_cast<uint16_t *>(ws + sp->l->blocks_off);
        int32_t *counts = reinterpret_cast<int32_t *>(ws + sp->l->counts_off);
        launch_sparse_select(qkv, 3 * H, qkv + H, 3 * H, V, sp->prefix_len, dims->heads, sp->tau, blocks, counts,
                             ws + sp->l->select_off, st);
        launch_sparse_attention(qkv, 3 * H, qkv + H, 3 * H, qkv + 2 * H, 3 * H, o, H, L_buf, V, sp->prefix_len,
                                dims->heads, 0.0f, blocks, counts, vt, st);
    }
    // 5 x1 = x + gate_a * (o W_o^T)
    launch_linear(o, H, w->w_o, H, w->b_o, x1, H, V, H, H, H3_EPI_RESIDUAL, x, H, gate_a, ldm, n_mod_groups, mod_idx,
                  st, part);
    launch_zero_rows(x1, H, H, V, L_buf, st);
    // 6 h2
    launch_modnorm(x1, H, nullptr, 0, shift_f, scale_f, nullptr, ldm, n_mod_groups, mod_idx, nullptr, 0, h2, H,
                   L_buf, V, (int32_t)H, dims->eps, dims->norm_type, st);
    // 7 g = silu(gate) * up
    launch_linear(h2, H, w->w_up, H, w->b_up, g, F, V, 2 * F, H, H3_EPI_SWIGLU, nullptr, 0, nullptr, 0, 1, nullptr,
                  st, part);
    launch_zero_rows(g, F, F, V, L_buf, st);
    // 8 y = x1 + gate_f * (g W_down^T)
    launch_linear(g, F, w->w_down, F, w->b_down, y, H, V, H, F, H3_EPI_RESIDUAL, x1, H, gate_f, ldm, n_mod_groups,
                  mod_idx, st, part);
    launch_zero_rows(y, H, H, V, L_buf, st);
    // 9 KV refresh export
    if (kv_export && kv_export->len > 0) {
        const h3_kv_export &e = *kv_export;
        launch_copy_rows(qkv + e.src_begin * 3 * H + H, 3 * H, e.k, e.ld, e.len, H, st);
        launch_copy_rows(qkv + e.src_begin * 3 * H + 2 * H, 3 * H, e.v, e.ld, e.len, H, st);
    }
}

}  // namespace
}  // namespace h3

using namespace h3;

extern "C" int h3_block_forward(const h3_dims *dims, const h3_block_weights *w, const uint16_t *x, uint16_t *y,
                                const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                const int32_t *pos, int64_t L_buf, int64_t valid_len, const h3_qgroup *groups,
                                int32_t n_groups, const h3_kv_export *kv_export, void *workspace,
                                size_t ws_bytes, void *stream) {
    int s = h3_check_block_forward(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len, groups,
                                   n_groups, kv_export, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    WsLayout l;
    ws_layout(dims, L_buf, groups, n_groups, &l);
    block_steps(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len, groups, n_groups, kv_export, l,
                workspace, nullptr, (hipStream_t)stream);
    return launch_status();
}

// A stack of blocks in place on x: every block's arguments are checked first,
// then the blocks run one after another on the stream, sharing the workspace
// (the AdaLN table cached per (block, step), Sol-H3 report §4.1).
extern "C" int h3_stack_forward(const h3_dims *dims, const h3_block_weights *w, int32_t n_blocks, uint16_t *x,
                                const float *mod, int64_t ld_mod_block, int32_t n_mod_groups,
                                const int32_t *mod_idx, const int32_t *pos, int64_t L_buf, int64_t valid_len,
                                void *workspace, size_t ws_bytes, void *stream) {
    int s = h3_check_stack_forward(dims, w, n_blocks, x, mod, ld_mod_block, n_mod_groups, mod_idx, pos, L_buf,
                                   valid_len, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0 || n_blocks == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    WsLayout l;
    ws_layout(dims, L_buf, nullptr, 0, &l);
    for (int32_t b = 0; b < n_blocks; ++b) {
        block_steps(dims, w + b, x, x, mod + (int64_t)b * ld_mod_block, n_mod_groups, mod_idx, pos, L_buf,
                    valid_len, nullptr, 0, nullptr, l, workspace, nullptr, (hipStream_t)stream);
        if ((s = launch_status()) != H3_OK) return s;
    }
    return H3_OK;
}

extern "C" int h3_block_forward_sparse(const h3_dims *dims, const h3_block_weights *w, const uint16_t *x,
                                       uint16_t *y, const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                       const int32_t *pos, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                       float tau, void *workspace, size_t ws_bytes, void *stream) {
    int s = h3_check_block_forward_sparse(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len,
                                          prefix_len, tau, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    BlockSparseLayout bl;
    block_sparse_layout(dims, L_buf, valid_len, prefix_len, &bl);
    const SparseStep sp{prefix_len, tau, &bl};
    block_steps(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len, nullptr, 0, nullptr, bl.base,
                workspace, &sp, (hipStream_t)stream);
    return launch_status();
}

// The MXFP8 block: the same steps with the four projections on MXFP8
// operands (Sol-H3 report, §3.3 "MXFP8 GEMM computation"), fed by the fused
// quantizing producers (modulate-norm and the SwiGLU epilogue) and, for the
// output projection, by a quantization of the BF16 attention output.
extern "C" int h3_block_forward_mxfp8(const h3_dims *dims, const h3_block_weights_mxfp8 *w, const uint16_t *x,
                                      uint16_t *y, const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                      const int32_t *pos, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                      float tau, void *workspace, size_t ws_bytes, void *stream) {
    int s = h3_check_block_forward_mxfp8(dims, w, x, y, mod, n_mod_groups, mod_idx, pos, L_buf, valid_len, prefix_len,
                                         tau, workspace, ws_bytes);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    MxWsLayout l;
    mx_ws_layout(dims, L_buf, valid_len, prefix_len, &l);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint8_t *hq = ws + l.off[H3_MXWS_HQ], *hs = ws + l.off[H3_MXWS_HS];
    uint16_t *qkv = reinterpret_cast<uint16_t *>(ws + l.off[H3_MXWS_QKV]);
    uint16_t *o = reinterpret_cast<uint16_t *>(ws + l.off[H3_MXWS_O]);
    uint8_t *oq = ws + l.off[H3_MXWS_OQ], *os = ws + l.off[H3_MXWS_OS];
    uint16_t *x1 = reinterpret_cast<uint16_t *>(ws + l.off[H3_MXWS_X1]);
    uint8_t *h2q = ws + l.off[H3_MXWS_H2Q], *h2s = ws + l.off[H3_MXWS_H2S];
    uint8_t *gq = ws + l.off[H3_MXWS_GQ], *gs = ws + l.off[H3_MXWS_GS];
    void *vt = ws + l.off[H3_MXWS_VT];

    const int64_t H = dims->hidden, F = dims->ffn, V = valid_len;
    const int64_t ldm = 6 * H;
    const float *shift_a = mod, *scale_a = mod + H, *gate_a = mod + 2 * H;
    const float *shift_f = mod + 3 * H, *scale_f = mod + 4 * H, *gate_f = mod + 5 * H;

    // 1 hq = MXFP8(modnorm(x))
    launch_modnorm_mx(x, H, nullptr, 0, shift_a, scale_a, nullptr, ldm, n_mod_groups, mod_idx, nullptr, 0, hq, H, hs,
                      L_buf, V, (int32_t)H, dims->eps, dims->norm_type, st);
    // 2 qkv
    launch_linear_mxfp8(hq, H, hs, L_buf, w->w_qkv, H, w->s_qkv, w->b_qkv, qkv, 3 * H, V, 3 * H, H, H3_EPI_STORE,
                        nullptr, 0, nullptr, 0, 1, nullptr, st);
    launch_zero_rows(qkv, 3 * H, 3 * H, V, L_buf, st);
    // 3 q~, k~
    launch_qk_norm_rope(qkv, qkv + H, 3 * H, w->q_gain, w->k_gain, pos, L_buf, V, dims->heads, dims->rot_dim,
                        dims->rope_pairing, dims->rope_theta, dims->eps, st);
    // 4 o (dense, or selection + list-mode attention), then oq = MXFP8(o)
    if (prefix_len >= 0 && prefix_len < V) {
        uint16_t *blocks = reinterpret_cast<uint16_t *>(ws + l.off[H3_MXWS_BLOCKS]);
        int32_t *counts = reinterpret_cast<int32_t *>(ws + l.off[H3_MXWS_COUNTS]);
        launch_sparse_select(qkv, 3 * H, qkv + H, 3 * H, V, prefix_len, dims->heads, tau, blocks, counts,
                             ws + l.off[H3_MXWS_SELECT], st);
        launch_sparse_attention(qkv, 3 * H, qkv + H, 3 * H, qkv + 2 * H, 3 * H, o, H, L_buf, V, prefix_len,
                                dims->heads, 0.0f, blocks, counts, vt, st);
    } else {
        launch_attention(qkv, 3 * H, qkv + H, 3 * H, qkv + 2 * H, 3 * H, o, H, L_buf, V, dims->heads, 0.0f, nullptr,
                         0, vt, st);
    }
    launch_mx_quantize(o, H, L_buf, V, H, oq, H, os, st);
    // 5 x1 = x + gate_a * (oq W_o^T)
    launch_linear_mxfp8(oq, H, os, L_buf, w->w_o, H, w->s_o, w->b_o, x1, H, V, H, H, H3_EPI_RESIDUAL, x, H, gate_a,
                        ldm, n_mod_groups, mod_idx, st);
    launch_zero_rows(x1, H, H, V, L_buf, st);
    // 6 h2q = MXFP8(modnorm(x1))
    launch_modnorm_mx(x1, H, nullptr, 0, shift_f, scale_f, nullptr, ldm, n_mod_groups, mod_idx, nullptr, 0, h2q, H,
                      h2s, L_buf, V, (int32_t)H, dims->eps, dims->norm_type, st);
    // 7 gq = MXFP8(silu(gate) * up), in the up-projection's epilogue
    launch_linear_mxfp8(h2q, H, h2s, L_buf, w->w_up, H, w->s_up, w->b_up, nullptr, 0, V, 2 * F, H, kEpiSwigluMx,
                        nullptr, 0, nullptr, 0, 1, nullptr, st, gq, F, gs, L_buf);
    launch_mx_zero_rows(gq, F, F, gs, L_buf, V, L_buf, st);
    // 8 y = x1 + gate_f * (gq W_down^T)
    launch_linear_mxfp8(gq, F, gs, L_buf, w->w_down, F, w->s_down, w->b_down, y, H, V, H, F, H3_EPI_RESIDUAL, x1, H,
                        gate_f, ldm, n_mod_groups, mod_idx, st);
    launch_zero_rows(y, H, H, V, L_buf, st);
    return launch_status();
}
