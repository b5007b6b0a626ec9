/*
 * h3block.h - C ABI of the MI355X (gfx950) forward pass of one MiniMax-H3 DiT
 * block over one long packed token sequence.
 *
 * Sources (cited by page title and section):
 *  [Sol-H3]   "Sol-H3: Recursive Self-Improvement for MiniMax-H3 Inference
 *             Acceleration on Sol-Engine across Cloud and Edge"
 *  [vLLM-H3]  "MiniMax H3 on vLLM-Omni: integrating FastVideo FastH3" (blog)
 *  [vflash]   vflash architecture notes, "choosing a memory strategy"
 *  [SolarWM]  "SolarWM H3 Realtime Interaction"
 *
 * Conventions shared by every entry point
 *  - BF16 tensors are passed as uint16_t bit patterns; FP32 as float.
 *  - Every matrix is row-major with an explicit row stride (ld, in elements).
 *  - Device pointers are HIP device (or managed) memory owned by the caller. The
 *    library allocates nothing, keeps no pointer after it returns and has no
 *    mutable state apart from a per-device cache of the architecture check.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work; buffers must stay alive until the stream has reached it.
 *  - A token buffer has L_buf rows of which the first valid_len are valid; rows
 *    [valid_len, L_buf) are the structural padding suffix ([vLLM-H3] §3.1: the
 *    attention backend receives the valid length and drops the suffix). Every
 *    output writes its padding rows as +0.0 and never reads padding inputs.
 *  - Every argument is validated on the host before anything is launched, so a
 *    call that returns an error has written nothing. H3_ERR_HIP means a HIP call
 *    failed after launches may have begun: the caller must treat the stream and
 *    its buffers as unusable (as [vflash] treats a failed worker's context).
 *  - Pointers to BF16 rows must be 16-byte aligned and row strides multiples of
 *    8 elements (128-bit loads), else H3_ERR_ALIGN.
 *  - Element offsets are computed in 64 bits wherever a buffer can exceed 2^31
 *    elements ([vflash]: widen large offsets before multiplying; the FFN-up
 *    output at 58,816 x 43,008 holds 2.53e9 elements).
 */
#ifndef H3BLOCK_H
#define H3BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3_ABI_VERSION 6
#define H3_MAX_SEGMENTS 4   /* K/V segments per query group */
#define H3_MAX_GROUPS 8     /* query groups per attention call */
#define H3_SPARSE_Q_BLOCK 256      /* block-sparse attention: target query block rows */
#define H3_SPARSE_K_BLOCK 64       /* block-sparse attention: target KV block rows    */
#define H3_SPARSE_MAX_KBLOCKS 4096 /* KV blocks per call (target rows <= 262,144)     */

enum h3_status {
    H3_OK = 0,
    H3_ERR_NULL = 1,        /* a required pointer is NULL                         */
    H3_ERR_SHAPE = 2,       /* sizes inconsistent or out of range                 */
    H3_ERR_UNSUPPORTED = 3, /* valid request this library does not implement      */
    H3_ERR_ALIGN = 4,       /* pointer not 16-B aligned or ld not a multiple of 8 */
    H3_ERR_ALIAS = 5,       /* buffers overlap in a way the call does not allow   */
    H3_ERR_WORKSPACE = 6,   /* workspace missing or too small                     */
    H3_ERR_DEVICE = 7,      /* current device is not an MI355X-class gfx950       */
    H3_ERR_HIP = 8          /* a HIP runtime call failed                          */
};

/* Width of one block. [Sol-H3] §3.5 gives hidden 5376; §3.2 (quantized
 * communication: a token/head record carries 3 x 128 QKV values) gives 128
 * channels per head, so 42 heads. */
typedef struct {
    int32_t hidden;       /* H = heads * head_dim                                 */
    int32_t heads;        /* attention heads                                      */
    int32_t head_dim;     /* channels per head; only 128 is accepted              */
    int32_t ffn;          /* F: SwiGLU width (w_up has 2F rows: gate | up);
                             multiple of 64                                       */
    int32_t rot_dim;      /* channels rotated by partial RoPE, multiple of 16,
                             0..head_dim                                          */
    int32_t norm_type;    /* 0 = RMSNorm (the pages' choice), 1 = LayerNorm       */
    int32_t rope_pairing; /* 0 = rotate-half pairs (i, i+rot/2); 1 = (2i, 2i+1)   */
    int32_t reserved;     /* must be 0                                            */
    float rope_theta;     /* RoPE base; omega_i = theta^(-2i/rot_dim)             */
    float eps;            /* epsilon of every norm                                */
} h3_dims;

/* Weights of one block, BF16, row-major [out, in]. Biases may be NULL.
 * w_qkv rows are q | k | v, each head-major (packed QKV, [Sol-H3] §3.2);
 * w_up rows are gate | up ([Sol-H3] §3.5 group (3): SwiGLU splitting). */
typedef struct {
    const uint16_t *w_qkv;  /* [3H, H] */
    const uint16_t *b_qkv;  /* [3H] or NULL */
    const uint16_t *q_gain; /* [head_dim], QK-norm gain shared by all heads */
    const uint16_t *k_gain; /* [head_dim] */
    const uint16_t *w_o;    /* [H, H] */
    const uint16_t *b_o;    /* [H] or NULL */
    const uint16_t *w_up;   /* [2F, H] */
    const uint16_t *b_up;   /* [2F] or NULL */
    const uint16_t *w_down; /* [H, F] */
    const uint16_t *b_down; /* [H] or NULL */
} h3_block_weights;

/* One K/V segment a query group attends over ([SolarWM] stages 2-3: video
 * queries read a pre-concatenated history K/V followed by the current chunk).
 * k == NULL selects rows [begin, begin+len) of the call's own K/V; otherwise
 * rows [begin, begin+len) of k and v, each [rows, heads*head_dim] with row
 * stride ld. Attention is non-causal; a group's keys are the concatenation of
 * its segments in order.
 * vt, kmax2: NULL, or (external segments only) the segment's V and key norms
 * already staged by h3_kv_stage over exactly these rows ([SolarWM] stage 3:
 * the history is prepared once at the KV refresh and reused by the chunk's
 * forwards); attention then reads them instead of staging V again. Both or
 * neither; the caller keeps them consistent with k and v. */
typedef struct {
    const uint16_t *k;
    const uint16_t *v;
    int64_t ld;
    int64_t begin;
    int64_t len;
    const uint16_t *vt;   /* [heads][128][round_up(len, 64)] BF16, 16-byte aligned */
    const float *kmax2;   /* [heads], 4-byte aligned */
} h3_kv_seg;

/* A query group: rows [q_begin, q_end) attend over n_seg segments. Groups must
 * be disjoint and lie inside [0, valid_len); valid rows outside every group are
 * written as zero. */
typedef struct {
    int64_t q_begin;
    int64_t q_end;
    int32_t n_seg;
    int32_t reserved;  /* must be 0 */
    h3_kv_seg seg[H3_MAX_SEGMENTS];
} h3_qgroup;

/* K/V refresh: copy the block's normalised, rotated K and its V for rows
 * [src_begin, src_begin+len) into k and v (row stride ld), so the next chunk's
 * forwards can read them as a history segment ([SolarWM] stage 3/4: the KV
 * refresh forward prepares the history for the following chunk). */
typedef struct {
    uint16_t *k;
    uint16_t *v;
    int64_t ld;
    int64_t src_begin;
    int64_t len;
} h3_kv_export;

/* ---------------------------------------------------------------------------
 * h3_block_forward - one DiT block ([Sol-H3] §3.5, its three operator groups
 * around the projections; [vLLM-H3] §3.1-3.2):
 *   h   = RMSNorm(x) * (1 + scale_a) + shift_a            group (1)
 *   qkv = h W_qkv^T (+ b_qkv)                              packed QKV
 *   q~, k~ = RoPE(RMSNorm_head(q) * q_gain), same for k    group (2)
 *   o   = softmax(q~ k~^T / sqrt(128)) v  per head, keys [0, valid_len) or per
 *         query group
 *   x1  = x + gate_a * (o W_o^T (+ b_o))                   group (1) residual
 *   h2  = RMSNorm(x1) * (1 + scale_f) + shift_f            group (1)
 *   g   = silu(u_gate) * u_up,  u = h2 W_up^T (+ b_up)     group (3)
 *   y   = x1 + gate_f * (g W_down^T (+ b_down));  y = 0 on padding rows
 * BF16 storage with FP32 arithmetic, FP32 modulation.
 *
 * x, y     [L_buf, hidden], ld = hidden. y == x is allowed (in place); any
 *          other overlap of y with x, the weights or the workspace is rejected.
 * mod      FP32 table [n_mod_groups, 6, hidden], rows per entry in the order
 *          shift_a, scale_a, gate_a, shift_f, scale_f, gate_f.
 * mod_idx  [L_buf] int32 table entry per row ("indexed" modulation), or NULL
 *          (entry 0 for every row). Indices are clamped into [0, n_mod_groups).
 * pos      [L_buf] int32 RoPE position per row, or NULL (position = row index);
 *          rows with a negative position are not rotated.
 * groups   NULL: dense attention of every valid row over keys [0, valid_len).
 *          Otherwise n_groups (1..H3_MAX_GROUPS) query groups.
 * kv_export NULL or one refresh copy (see h3_kv_export).
 * workspace device memory of at least
 *          h3_block_workspace_bytes(dims, L_buf, groups, n_groups) bytes,
 *          256-byte aligned. After the call it holds the block's intermediates at
 *          the offsets h3_block_workspace_layout reports.
 * ------------------------------------------------------------------------- */
int h3_block_forward(const h3_dims *dims, const h3_block_weights *w,
                     const uint16_t *x, uint16_t *y,
                     const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                     const int32_t *pos, int64_t L_buf, int64_t valid_len,
                     const h3_qgroup *groups, int32_t n_groups,
                     const h3_kv_export *kv_export,
                     void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * h3_stack_forward - n_blocks DiT blocks applied in order to one packed
 * sequence, in place: x <- block_{n-1}( ... block_1(block_0(x)) ), each block
 * exactly as h3_block_forward with dense attention over [0, valid_len). This
 * is one denoiser forward of a step; the step's modulation comes from the
 * precomputed AdaLN table cached per (block, step) ([Sol-H3] §4.1 "AdaLN
 * precompute"), of which the caller passes the step's slice.
 *
 * w        [n_blocks] weight sets (block b uses w[b]).
 * x        [L_buf, hidden], ld = hidden; input and, on return, output.
 * mod      block b reads its FP32 table [n_mod_groups, 6, hidden] at
 *          mod + b * ld_mod_block (floats); ld_mod_block >= 0 and a multiple
 *          of 4 (16-byte aligned tables). For a table [blocks][steps][6][H],
 *          step s passes mod + s * 6H and ld_mod_block = steps * 6H.
 * mod_idx, pos, L_buf, valid_len: as h3_block_forward, shared by every block.
 * workspace h3_block_workspace_bytes(dims, L_buf, NULL, 0) bytes, reused by
 *          every block; on return it holds the last block's intermediates.
 * Every block's arguments are checked before the first launch, so a rejected
 * call writes nothing. n_blocks == 0 returns H3_OK without work.
 * ------------------------------------------------------------------------- */
int h3_stack_forward(const h3_dims *dims, const h3_block_weights *w, int32_t n_blocks,
                     uint16_t *x, const float *mod, int64_t ld_mod_block,
                     int32_t n_mod_groups, const int32_t *mod_idx,
                     const int32_t *pos, int64_t L_buf, int64_t valid_len,
                     void *workspace, size_t ws_bytes, void *stream);

/* Workspace size of h3_block_forward for L_buf rows and the given query groups
 * (NULL for dense attention), in bytes. Returns 0 on invalid arguments. */
size_t h3_block_workspace_bytes(const h3_dims *dims, int64_t L_buf,
                                const h3_qgroup *groups, int32_t n_groups);

/* Intermediates h3_block_forward leaves in its workspace, as byte offsets and
 * row strides (elements). All are BF16 [L_buf, cols] with padding rows zero:
 *   H3_WS_H   h   (cols H)      H3_WS_QKV qkv (cols 3H; q~ | k~ | v after
 *   H3_WS_O   o   (cols H)                  QK-norm and RoPE)
 *   H3_WS_X1  x1  (cols H)      H3_WS_H2  h2  (cols H)
 *   H3_WS_G   g   (cols F)
 *   H3_WS_VT  attention's V^T staging (see h3_attention_workspace_bytes);
 *             its "row stride" entry holds its size in bytes.
 *   H3_WS_GEMM the projections' workspace (stream-K partial sums and tile
 *             counters, see h3_linear_workspace_bytes), the largest any of
 *             the four needs at up to L_buf rows; its "row stride" entry
 *             holds its size in bytes (0 when none needs any).           */
enum { H3_WS_H = 0, H3_WS_QKV = 1, H3_WS_O = 2, H3_WS_X1 = 3, H3_WS_H2 = 4, H3_WS_G = 5,
       H3_WS_VT = 6, H3_WS_GEMM = 7, H3_WS_COUNT = 8 };
int h3_block_workspace_layout(const h3_dims *dims, int64_t L_buf,
                              const h3_qgroup *groups, int32_t n_groups,
                              int64_t offsets[H3_WS_COUNT], int64_t lds[H3_WS_COUNT]);

/* ---------------------------------------------------------------------------
 * h3_attention - exact multi-head attention over a packed sequence
 * ([Sol-H3] §3.2 dense SDPA attention over the packed QKV, flat
 * (total, heads, head_dim) layout; [vLLM-H3] §3.1 valid length; [SolarWM]
 * stage 2 grouped queries):
 *   o[r, h] = sum_t softmax_t(q[r,h] . k[t,h] * scale) v[t,h]
 * q, k, v  [L_buf, heads*head_dim] BF16 at row strides ld_q, ld_k, ld_v (they
 *          may be column blocks of one packed qkv buffer).
 * o        [L_buf, heads*head_dim] BF16 at ld_o; must not overlap q, k or v.
 * softmax_scale 0 selects 1/sqrt(head_dim).
 * groups   NULL: every row in [0, valid_len) attends over keys [0, valid_len).
 * FP32 scores, softmax and accumulation; P is rounded to BF16 for the P.V
 * product. Padding rows and valid rows outside every group are written 0.
 * workspace device memory of at least h3_attention_workspace_bytes(...) bytes,
 *          256-byte aligned: each distinct K/V segment's V is first staged
 *          there transposed per head ([heads][128][keys rounded up to 64]).
 * ------------------------------------------------------------------------- */
int h3_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                 const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o,
                 int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                 float softmax_scale, const h3_qgroup *groups, int32_t n_groups,
                 void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes h3_attention needs: for every distinct segment (dense: the
 * valid rows) not staged by h3_kv_stage, heads * 128 * round_up(len, 64) BF16
 * values; then the partial records of query tiles cut into key-range pieces,
 * the per-head key norm maxima, one int32 per work item (the items left to
 * the online-softmax form) and 256 bytes of work-queue counters, each area
 * 256-byte aligned. The call clears or writes all of it before reading it.
 * 0 on bad input. */
size_t h3_attention_workspace_bytes(int64_t valid_len, int32_t heads,
                                    const h3_qgroup *groups, int32_t n_groups);

/* ---------------------------------------------------------------------------
 * h3_kv_stage - prepare an external K/V segment once for the attention calls
 * that will read it ([SolarWM] stage 3: the KV refresh prepares the history
 * K/V for the following chunk's forwards): rows [0, len) of k and v
 * ([len, heads*128] at row stride ld) give
 *   vt     [heads][128][round_up(len, 64)] BF16: V transposed per head, keys
 *          permuted inside each 16-key group and zero past len, exactly as
 *          attention stages V itself (h3_kv_stage_bytes(len, heads) bytes);
 *   kmax2  [heads] FP32: the largest squared norm of a key row per head.
 * Pass them in an h3_kv_seg (with k + begin * ld ... as that segment's rows)
 * as vt and kmax2. vt and kmax2 must not overlap k, v or each other.
 * ------------------------------------------------------------------------- */
int h3_kv_stage(const uint16_t *k, const uint16_t *v, int64_t ld, int64_t len, int32_t heads, int32_t head_dim,
                uint16_t *vt, float *kmax2, void *stream);
size_t h3_kv_stage_bytes(int64_t len, int32_t heads);
int h3_check_kv_stage(const uint16_t *k, const uint16_t *v, int64_t ld, int64_t len, int32_t heads,
                      int32_t head_dim, const uint16_t *vt, const float *kmax2);

/* ---------------------------------------------------------------------------
 * h3_attention_noalloc - h3_attention for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and result, with no workspace
 * argument. The workspace is a fixed device array inside the library, one per
 * GPU, of H3_ATTENTION_SCRATCH_BYTES bytes, held until the process ends.
 * The call allocates nothing and calls no allocating routine.
 *
 * Limit: h3_attention_workspace_bytes(valid_len, heads, groups, n_groups)
 * must not exceed H3_ATTENTION_SCRATCH_BYTES (128 MiB: at 42 heads, dense
 * attention up to 6,144 valid rows, e.g. the 4,096-token full-width block),
 * else H3_ERR_WORKSPACE and nothing is launched. Other errors as h3_attention.
 * Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined results.
 * ------------------------------------------------------------------------- */
#define H3_ATTENTION_SCRATCH_BYTES (128ll << 20)
int h3_attention_noalloc(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                         const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o,
                         int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                         float softmax_scale, const h3_qgroup *groups, int32_t n_groups,
                         void *stream);

/* ---------------------------------------------------------------------------
 * h3_fused_modulate_norm - operator group (1) of [Sol-H3] §3.5 (residual
 * addition with indexed gating, RMSNorm, indexed scale/shift modulation), the
 * merged FP32 modulation + norm + residual of [vLLM-H3] §3.2:
 *   if branch: x1 = bf16(x + gate[i] * branch), written to x1_out; z = x1
 *   else:      z = x
 *   h = bf16(norm(z) * (1 + scale[i]) + shift[i]),  i = mod_idx[r] or 0
 * x, branch, x1_out, h_out: [L_buf, hidden] BF16 at their ld. x1_out may equal
 * x (in place); h_out must not overlap the inputs.
 * shift, scale, gate: FP32 [G][hidden] with ld_mod_group floats between table
 * entries (6*hidden for the block's [G, 6, hidden] table). gate may be NULL
 * when branch is NULL. Indices are clamped into [0, n_mod_groups).
 * norm_type 0 = RMSNorm z / sqrt(mean z^2 + eps); 1 = LayerNorm with the
 * population variance. hidden <= 16384, multiple of 8.
 * ------------------------------------------------------------------------- */
int h3_fused_modulate_norm(const uint16_t *x, int64_t ld_x,
                           const uint16_t *branch, int64_t ld_b,
                           const float *shift, const float *scale, const float *gate,
                           int64_t ld_mod_group, int32_t n_mod_groups, const int32_t *mod_idx,
                           uint16_t *x1_out, int64_t ld_x1, uint16_t *h_out, int64_t ld_h,
                           int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                           int32_t norm_type, void *stream);

/* ---------------------------------------------------------------------------
 * h3_qk_norm_rope - operator group (2) of [Sol-H3] §3.5 (QK normalization with
 * partial RoPE), the fused Q/K RMSNorm + RoPE of [vLLM-H3] §3.2, in place:
 *   per row r and head j: t = RMSNorm(t[r, j*128 : j*128+128]) * gain
 *   then rotate the first rot_dim channels by phi_i = pos[r] * theta^(-2i/rot)
 *   (pairing 0: channels (i, i + rot/2); pairing 1: (2i, 2i+1)):
 *   (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi)
 * q, k     [L_buf, heads*128] BF16 at row stride ld (3*hidden when they are
 *          the column blocks of a packed qkv buffer). Padding rows are zeroed.
 * pos      [L_buf] int32 or NULL (= row index); negative: no rotation.
 * The angle and its sine/cosine are computed in FP64 and rounded to FP32, so
 * rows at positions near 6e4 keep full accuracy.
 * ------------------------------------------------------------------------- */
int h3_qk_norm_rope(uint16_t *q, uint16_t *k, int64_t ld,
                    const uint16_t *q_gain, const uint16_t *k_gain, const int32_t *pos,
                    int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                    int32_t rot_dim, int32_t pairing, float theta, float eps, void *stream);

/* ---------------------------------------------------------------------------
 * h3_swiglu - operator group (3) of [Sol-H3] §3.5 (SwiGLU splitting, SiLU,
 * multiplication), the fused SwiGLU of [vLLM-H3] §3.2:
 *   g[r, j] = bf16(silu(u[r, j]) * u[r, ffn + j]),  silu(z) = z / (1 + e^-z)
 * u [L_buf, 2*ffn] BF16 at ld_u; g [L_buf, ffn] BF16 at ld_g, not overlapping u.
 * ------------------------------------------------------------------------- */
int h3_swiglu(const uint16_t *u, int64_t ld_u, uint16_t *g, int64_t ld_g,
              int64_t L_buf, int64_t valid_len, int32_t ffn, void *stream);

/* ---------------------------------------------------------------------------
 * Precision-preserving LoRA consumer fusion ([Sol-H3] §3.5 "Precision-
 * preserving LoRA fusion" and Appendix B): the base projection output and the
 * LoRA branch's output delta stay separate (the three GEMMs are unchanged) and
 * their sum is never stored: the consumer forms s = bf16(base + delta), round
 * to nearest even, and then runs exactly as its plain entry point does on s.
 * The result is bit-identical to storing bf16(base + delta) and calling the
 * plain entry point on it. delta has the shape of base, at its own row
 * stride, and must not overlap any output. Padding rows follow the plain
 * entry point.
 *
 * h3_qk_norm_rope_lora: the QKV consumer (QK normalization, RoPE, packing):
 *   q := qk_norm_rope(bf16(q + dq)), k likewise with dk (as h3_qk_norm_rope);
 *   v := bf16(v + dv) when v is not NULL (dv then required). q, k, v share
 *   the row stride ld (the column blocks of a packed qkv buffer); dq, dk, dv
 *   share ld_d.
 * ------------------------------------------------------------------------- */
int h3_qk_norm_rope_lora(uint16_t *q, uint16_t *k, uint16_t *v, int64_t ld,
                         const uint16_t *dq, const uint16_t *dk, const uint16_t *dv, int64_t ld_d,
                         const uint16_t *q_gain, const uint16_t *k_gain, const int32_t *pos,
                         int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                         int32_t rot_dim, int32_t pairing, float theta, float eps, void *stream);

/* h3_fused_modulate_norm_lora: the residual-modulation consumer. branch,
 * delta and gate are required; s = bf16(branch + delta), then
 *   gate_bf16 == 0: x1 = bf16(x + gate[i] * s)
 *   gate_bf16 != 0: x1 = bf16(x + bf16(gate[i] * s))   (the final FFN
 *                   consumer, which keeps the intermediate BF16 gate product)
 *   h = bf16(norm(x1) * (1 + scale[i]) + shift[i]) as h3_fused_modulate_norm;
 * h_out may be NULL (residual only; shift and scale are then not read). */
int h3_fused_modulate_norm_lora(const uint16_t *x, int64_t ld_x,
                                const uint16_t *branch, int64_t ld_b, const uint16_t *delta, int64_t ld_d,
                                const float *shift, const float *scale, const float *gate,
                                int64_t ld_mod_group, int32_t n_mod_groups, const int32_t *mod_idx,
                                uint16_t *x1_out, int64_t ld_x1, uint16_t *h_out, int64_t ld_h,
                                int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                int32_t norm_type, int32_t gate_bf16, void *stream);

/* h3_swiglu_lora: the SwiGLU consumer. du [L_buf, 2*ffn] at ld_du:
 *   g[r, j] = bf16(silu(s[r, j]) * s[r, ffn + j]),  s = bf16(u + du). */
int h3_swiglu_lora(const uint16_t *u, int64_t ld_u, const uint16_t *du, int64_t ld_du,
                   uint16_t *g, int64_t ld_g, int64_t L_buf, int64_t valid_len, int32_t ffn, void *stream);

/* ---------------------------------------------------------------------------
 * h3_linear - the block's projections as one BF16 MFMA GEMM with FP32
 * accumulation, c = a W^T (+ bias), W stored [N, K] ([Sol-H3] §3.2 packed QKV
 * projection; §3.5 group (1) gated residual and group (3) SwiGLU as epilogues):
 *   H3_EPI_STORE    c[r, n] = bf16(acc + bias[n])                (N columns)
 *   H3_EPI_RESIDUAL c[r, n] = bf16(resid[r, n] + gate[i][n] * (acc + bias[n]))
 *   H3_EPI_SWIGLU   W has N = 2F rows (gate | up); c has F columns:
 *                   c[r, j] = bf16(silu(acc_j + b_j) * (acc_{F+j} + b_{F+j}))
 * a [M_buf, K] at lda; rows [M_valid, M_buf) of c are written 0.
 * resid: [M_buf, N] at ld_r (H3_EPI_RESIDUAL; may equal c for in place).
 * gate: FP32 [G][N] with ld_gate_group floats between entries; i = mod_idx[r]
 * or 0, clamped into [0, n_mod_groups).
 * K must be a multiple of 64 (else H3_ERR_UNSUPPORTED); N a multiple of 8
 * (SwiGLU: N a multiple of 16). gate's ld_gate_group must be a multiple of 4.
 * ------------------------------------------------------------------------- */
enum { H3_EPI_STORE = 0, H3_EPI_RESIDUAL = 1, H3_EPI_SWIGLU = 2 };
int h3_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw,
              const uint16_t *bias, uint16_t *c, int64_t ldc,
              int64_t M_buf, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
              const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
              int32_t n_mod_groups, const int32_t *mod_idx,
              void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes h3_linear uses for M_valid rows: 0 when it needs none.
 * With a workspace of at least this size (256-byte aligned, overlapping no
 * operand):
 *  - the tiles of a last, partial round that fills at most 4/5 of the chip's
 *    256 workgroup slots, and leaves idle slot time worth at least 55 K
 *    stages of 64 (K/64 x the idle share), are cut into equal ranges of K
 *    stages over all slots (stream-K tail); each range leaves FP32 partial
 *    sums there and a fix-up pass adds them in K order and applies the
 *    epilogue;
 *  - when the other tiles fill at least 8 rounds of the slots, the last
 *    twelfth of each XCD's share of them (at least 96) is drawn at run time
 *    from per-XCD counters kept in the 256 bytes after the partial sums, so
 *    that XCDs running faster under load take over the end of slower ones'
 *    shares. The counters are cleared inside the call.
 * The result does not depend on the workspace beyond the FP32 summation
 * order of split tiles. workspace NULL: one workgroup per tile, taken by
 * workgroup index. A non-NULL workspace smaller than this size is
 * H3_ERR_WORKSPACE. Calls that overlap in time must not share a workspace. */
size_t h3_linear_workspace_bytes(int64_t M_valid, int64_t N, int64_t K, int32_t epilogue);

/* ---------------------------------------------------------------------------
 * Sol-Attn block-sparse attention ([Sol-H3] §3.4 "Sparse Attention").
 *
 * The packed sequence is [prefix | target]: rows [0, P) are the prefix
 * (text, conditioning video and audio), rows [P, valid_len) the target video.
 * Target rows are cut into query blocks of H3_SPARSE_Q_BLOCK rows and target
 * keys into KV blocks of H3_SPARSE_K_BLOCK rows, both counted from P; the
 * last block of each may be short. n_qb = ceil(T / 256), n_kb = ceil(T / 64),
 * T = valid_len - P <= H3_SPARSE_MAX_KBLOCKS * 64 (else H3_ERR_UNSUPPORTED).
 * The block sizes are this library's choice; the pages do not give them.
 *
 * h3_sparse_select - the block selection. For head h and query block b:
 *   s_bj = mean(q rows of b) . mean(k rows of j) / sqrt(128)  (j over the
 *          target KV blocks; q, k after Q/K RMSNorm and RoPE)
 *   j is selected when s_bj > mu_b + tau * sigma_b, mu_b and sigma_b being
 *   the mean and the population standard deviation of s_b. over j.
 * Everything is FP32. A larger tau selects fewer blocks.
 * q, k     [valid_len, heads*128] BF16 at ld_q, ld_k (the column blocks of a
 *          packed qkv buffer after h3_qk_norm_rope).
 * blocks   out, uint16 [heads][n_qb][n_kb]: row (h, b) starts with the
 *          selected j in ascending order; the rest of the row is unspecified.
 * counts   out, int32 [heads][n_qb]: the number of selected blocks.
 * workspace device memory of h3_sparse_select_workspace_bytes(...) bytes,
 *          256-byte aligned (the pooled means, FP32).
 * blocks, counts and the workspace must not overlap each other, q or k.
 * T == 0 is a no-op.
 * ------------------------------------------------------------------------- */
int h3_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                     int64_t valid_len, int64_t prefix_len, int32_t heads, int32_t head_dim, float tau,
                     uint16_t *blocks, int32_t *counts, void *workspace, size_t ws_bytes, void *stream);
/* Workspace bytes of h3_sparse_select (0 when T == 0 or on bad input). */
size_t h3_sparse_select_workspace_bytes(int64_t valid_len, int64_t prefix_len, int32_t heads);

/* h3_sparse_attention - attention with the selected blocks:
 *   prefix rows r < P:  o[r] = softmax over every key in [0, valid_len)
 *   target rows of query block b: o[r] = softmax over the prefix keys [0, P)
 *       (always attended, exactly) and the keys of the KV blocks listed in
 *       blocks[h][b][0 .. counts[h][b])
 * i.e. dense attention masked to the selected blocks, with the arithmetic of
 * h3_attention (FP32 scores and softmax, BF16 P). q, k, v, o and
 * softmax_scale as in h3_attention; padding rows of o are written 0.
 * P must be >= 1 when valid_len > P. blocks / counts as h3_sparse_select
 * writes them (any source is accepted): counts are clamped into [0, n_kb];
 * list entries >= n_kb contribute nothing; an entry listed twice counts twice.
 * Lists are read, never written.
 * workspace: h3_sparse_attention_workspace_bytes(...) bytes, 256-byte aligned
 *          (V^T staging of the prefix and the target keys).
 * valid_len == P falls back to dense attention over [0, valid_len).
 * ------------------------------------------------------------------------- */
int h3_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                        const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o,
                        int64_t L_buf, int64_t valid_len, int64_t prefix_len, int32_t heads, int32_t head_dim,
                        float softmax_scale, const uint16_t *blocks, const int32_t *counts,
                        void *workspace, size_t ws_bytes, void *stream);
size_t h3_sparse_attention_workspace_bytes(int64_t valid_len, int64_t prefix_len, int32_t heads);

/* h3_block_forward_sparse - h3_block_forward with step 4 replaced by Sol-Attn
 * block-sparse attention ([Sol-H3] §3.4): after QK-norm and RoPE, the block
 * runs h3_sparse_select on its own q~, k~ with threshold tau, then
 * h3_sparse_attention with prefix_len (prefix rows dense, prefix keys always
 * attended). The pages keep the first two layers dense and use tau 1.0, 1.25
 * and 1.5 over the three refinement steps: that schedule belongs to the
 * caller, which picks this entry point or h3_block_forward per layer.
 * Arguments as h3_block_forward (no query groups, no K/V export), plus
 * prefix_len (>= 1 when valid_len > prefix_len) and a finite tau.
 * workspace: h3_block_sparse_workspace_bytes(dims, L_buf, valid_len,
 *          prefix_len) bytes, 256-byte aligned. It begins with the dense
 *          block's layout (h3_block_workspace_layout(dims, L_buf, NULL, 0)
 *          gives the intermediates' offsets); the V^T slot may be larger,
 *          and the selection's lists, counts and pooled means follow it. */
int h3_block_forward_sparse(const h3_dims *dims, const h3_block_weights *w,
                            const uint16_t *x, uint16_t *y,
                            const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                            const int32_t *pos, int64_t L_buf, int64_t valid_len,
                            int64_t prefix_len, float tau,
                            void *workspace, size_t ws_bytes, void *stream);
size_t h3_block_sparse_workspace_bytes(const h3_dims *dims, int64_t L_buf, int64_t valid_len,
                                       int64_t prefix_len);
/* Byte offsets, inside that workspace, of the selection the call made: the
 * block lists (uint16 [heads][n_qb][n_kb]) and their counts (int32
 * [heads][n_qb]), as h3_sparse_select documents them. */
int h3_block_sparse_workspace_layout(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                     int64_t *blocks_off, int64_t *counts_off);

/* ---------------------------------------------------------------------------
 * MXFP8 GEMMs ([Sol-H3] §3.3 "Compute Quantization", "MXFP8 GEMM
 * computation"): E4M3 values with one E8M0 scale per 32 consecutive values
 * along the reduction dimension K. The pages name the formats; the scale of
 * a group is chosen by the microscaling rule (this library's reading): with
 * amax the group's largest magnitude, the shared exponent is
 * e = floor(log2 amax) - 8 (clamped to >= -127; an all-zero group takes
 * -127), the scale code is e + 127, and each element is x * 2^-e rounded to
 * the nearest E4M3 value (ties to even) with magnitudes above 448 saturating
 * to 448. E4M3 is the 1-4-3 format with bias 7, no infinities, largest
 * finite value 448.
 *
 * MXFP8 matrix [rows, K] (K a multiple of 128): codes, uint8 [rows][ld]
 * (ld >= K, a multiple of 16, 16-byte aligned base), plus scales, uint8
 * [K / 128][scale_rows][4] (4-byte aligned): byte (g / 4, r, g % 4) is the
 * scale code of row r's k group g (k in [32 g, 32 g + 32)). scale_rows is the
 * row count of the scale array (>= the rows in use). The pages' scale
 * buffers use cuBLASLt's SWIZZLE_32_4_4 layout; this layout instead puts one
 * K stage's scales for a tile of rows in one contiguous run, which is what
 * the gfx950 kernel loads.
 *
 * h3_mxfp8_quantize: x [rows_buf, K] BF16 at ld_x -> codes q at ld_q and
 * scales (scale_rows = rows_buf). Rows [rows_valid, rows_buf) get zero codes
 * and zero scale codes; x's padding rows are not read. K % 128 != 0 is
 * H3_ERR_UNSUPPORTED. Outputs must not overlap x or each other.
 * ------------------------------------------------------------------------- */
int h3_mxfp8_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K,
                      uint8_t *q, int64_t ld_q, uint8_t *scales, void *stream);

/* h3_linear_mxfp8: c = dequant(a) dequant(w)^T (+ bias) with h3_linear's
 * epilogues (STORE, RESIDUAL, SWIGLU; same arguments, BF16 output, rows
 * [M_valid, M_buf) of c written 0). a: MXFP8 [M_buf, K] with scale_rows
 * a_scale_rows (>= M_valid); w: MXFP8 [N, K] with scale_rows N. Products are
 * exact and accumulated in FP32 on gfx950's scaled MFMA. K must be a
 * multiple of 128 (else H3_ERR_UNSUPPORTED); N a multiple of 8 (16 for
 * SwiGLU). c must not overlap any input but resid (which may equal it). */
int h3_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                    const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias,
                    uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                    int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                    int64_t ld_gate_group, int32_t n_mod_groups, const int32_t *mod_idx, void *stream);

/* h3_fused_modulate_norm_mxfp8: h3_fused_modulate_norm whose output h is
 * written as MXFP8 straight from its FP32 values (the fused quantizing
 * producer of [Sol-H3] §3.3): codes hq [L_buf, hidden] at ld_hq and scales
 * hs with L_buf scale rows; no BF16 h exists. hidden must be a multiple of
 * 128 (else H3_ERR_UNSUPPORTED). Padding rows get zero codes and scale
 * codes. The optional residual (branch, gate, x1_out) is as in
 * h3_fused_modulate_norm. */
int h3_fused_modulate_norm_mxfp8(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                 const float *shift, const float *scale, const float *gate,
                                 int64_t ld_mod_group, int32_t n_mod_groups, const int32_t *mod_idx,
                                 uint16_t *x1_out, int64_t ld_x1, uint8_t *hq, int64_t ld_hq, uint8_t *hs,
                                 int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                 int32_t norm_type, void *stream);

/* Weights of one block in MXFP8 (each made by h3_mxfp8_quantize of the BF16
 * weight with rows_buf = rows_valid = its row count): codes with row stride
 * equal to K, scales with scale_rows equal to the weight's row count.
 * Biases and QK-norm gains stay BF16. */
typedef struct {
    const uint8_t *w_qkv, *s_qkv;   /* [3H, H] */
    const uint8_t *w_o, *s_o;       /* [H, H] */
    const uint8_t *w_up, *s_up;     /* [2F, H], gate | up */
    const uint8_t *w_down, *s_down; /* [H, F] */
    const uint16_t *b_qkv, *b_o, *b_up, *b_down;  /* or NULL */
    const uint16_t *q_gain, *k_gain;
} h3_block_weights_mxfp8;

/* h3_block_forward_mxfp8 - the block of h3_block_forward with its four
 * projections as MXFP8 GEMMs ([Sol-H3] §3.3: attention and FFN projections in
 * MXFP8, fed by fused quantizing producers):
 *   hq  = MXFP8(modnorm(x))            (fused producer, from FP32 values)
 *   qkv = bf16(dequant(hq) dequant(W_qkv)^T + b)
 *   q~, k~ as h3_block_forward; o = attention (BF16)
 *   oq  = MXFP8(o)                     (h3_mxfp8_quantize of the BF16 o)
 *   x1  = bf16(x + gate_a * (dequant(oq) dequant(W_o)^T + b))
 *   h2q = MXFP8(modnorm(x1))           (fused producer)
 *   gq  = MXFP8(silu(u_gate) * u_up), u = dequant(h2q) dequant(W_up)^T + b
 *                                      (fused into the up-projection epilogue)
 *   y   = bf16(x1 + gate_f * (dequant(gq) dequant(W_down)^T + b)); 0 on padding
 * Attention: dense over [0, valid_len) when prefix_len < 0; otherwise Sol-Attn
 * block-sparse attention as in h3_block_forward_sparse (prefix rows
 * [0, prefix_len) dense, target rows block-sparse with threshold tau): the
 * pages run their refinement blocks with both. No query groups, no K/V
 * export. hidden and ffn must be multiples of 128. Other arguments as
 * h3_block_forward. The quantization is approximate: the result differs from
 * the BF16 block by the MXFP8 rounding of the four GEMMs' operands.
 * workspace: h3_block_mxfp8_workspace_bytes(dims, L_buf, valid_len,
 *          prefix_len) bytes, 256-byte aligned; h3_block_mxfp8_workspace_layout
 *          gives the offsets of the intermediates it holds after the call. */
enum { H3_MXWS_HQ = 0, H3_MXWS_HS = 1, H3_MXWS_QKV = 2, H3_MXWS_O = 3, H3_MXWS_OQ = 4, H3_MXWS_OS = 5,
       H3_MXWS_X1 = 6, H3_MXWS_H2Q = 7, H3_MXWS_H2S = 8, H3_MXWS_GQ = 9, H3_MXWS_GS = 10, H3_MXWS_VT = 11,
       H3_MXWS_BLOCKS = 12, H3_MXWS_COUNTS = 13, H3_MXWS_SELECT = 14, H3_MXWS_COUNT = 15 };
int h3_block_forward_mxfp8(const h3_dims *dims, const h3_block_weights_mxfp8 *w,
                           const uint16_t *x, uint16_t *y,
                           const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                           const int32_t *pos, int64_t L_buf, int64_t valid_len,
                           int64_t prefix_len, float tau,
                           void *workspace, size_t ws_bytes, void *stream);
size_t h3_block_mxfp8_workspace_bytes(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len);
/* Byte offsets of the intermediates (codes [L_buf, cols] with row stride
 * cols; scales [cols / 128][L_buf][4]; BF16 qkv [L_buf, 3H], o and x1
 * [L_buf, H] with row strides 3H and H; the V^T staging area; with sparse
 * attention the selection's lists and counts, as h3_sparse_select writes
 * them, and its pooled means). */
int h3_block_mxfp8_workspace_layout(const h3_dims *dims, int64_t L_buf, int64_t valid_len, int64_t prefix_len,
                                    int64_t offsets[H3_MXWS_COUNT]);

/* Host-only validators: the same checks each entry point runs before it
 * launches anything, callable without a GPU. They return an h3_status. */
int h3_check_block_forward(const h3_dims *dims, const h3_block_weights *w,
                           const uint16_t *x, uint16_t *y,
                           const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                           const int32_t *pos, int64_t L_buf, int64_t valid_len,
                           const h3_qgroup *groups, int32_t n_groups,
                           const h3_kv_export *kv_export,
                           const void *workspace, size_t ws_bytes);
int h3_check_stack_forward(const h3_dims *dims, const h3_block_weights *w, int32_t n_blocks,
                           const uint16_t *x, const float *mod, int64_t ld_mod_block,
                           int32_t n_mod_groups, const int32_t *mod_idx,
                           const int32_t *pos, int64_t L_buf, int64_t valid_len,
                           const void *workspace, size_t ws_bytes);
int h3_check_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                       const uint16_t *v, int64_t ld_v, const uint16_t *o, int64_t ld_o,
                       int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                       float softmax_scale, const h3_qgroup *groups, int32_t n_groups,
                       const void *workspace, size_t ws_bytes);
int h3_check_fused_modulate_norm(const uint16_t *x, int64_t ld_x,
                                 const uint16_t *branch, int64_t ld_b,
                                 const float *shift, const float *scale, const float *gate,
                                 int64_t ld_mod_group, int32_t n_mod_groups,
                                 const uint16_t *x1_out, int64_t ld_x1,
                                 const uint16_t *h_out, int64_t ld_h,
                                 int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                 int32_t norm_type);
int h3_check_qk_norm_rope(const uint16_t *q, const uint16_t *k, int64_t ld,
                          const uint16_t *q_gain, const uint16_t *k_gain,
                          int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                          int32_t rot_dim, int32_t pairing, float theta, float eps);
int h3_check_swiglu(const uint16_t *u, int64_t ld_u, const uint16_t *g, int64_t ld_g,
                    int64_t L_buf, int64_t valid_len, int32_t ffn);
int h3_check_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw,
                    const uint16_t *bias, const uint16_t *c, int64_t ldc, int64_t M_buf,
                    int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                    const uint16_t *resid, int64_t ld_r, const float *gate,
                    int64_t ld_gate_group, int32_t n_mod_groups,
                    const void *workspace, size_t ws_bytes);

int h3_check_qk_norm_rope_lora(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t ld,
                               const uint16_t *dq, const uint16_t *dk, const uint16_t *dv, int64_t ld_d,
                               const uint16_t *q_gain, const uint16_t *k_gain,
                               int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                               int32_t rot_dim, int32_t pairing, float theta, float eps);
int h3_check_fused_modulate_norm_lora(const uint16_t *x, int64_t ld_x,
                                      const uint16_t *branch, int64_t ld_b, const uint16_t *delta, int64_t ld_d,
                                      const float *shift, const float *scale, const float *gate,
                                      int64_t ld_mod_group, int32_t n_mod_groups,
                                      const uint16_t *x1_out, int64_t ld_x1,
                                      const uint16_t *h_out, int64_t ld_h,
                                      int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                      int32_t norm_type, int32_t gate_bf16);
int h3_check_swiglu_lora(const uint16_t *u, int64_t ld_u, const uint16_t *du, int64_t ld_du,
                         const uint16_t *g, int64_t ld_g, int64_t L_buf, int64_t valid_len, int32_t ffn);

int h3_check_block_forward_sparse(const h3_dims *dims, const h3_block_weights *w,
                                  const uint16_t *x, uint16_t *y,
                                  const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                  const int32_t *pos, int64_t L_buf, int64_t valid_len,
                                  int64_t prefix_len, float tau, const void *workspace, size_t ws_bytes);
int h3_check_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                           int64_t valid_len, int64_t prefix_len, int32_t heads, int32_t head_dim, float tau,
                           const uint16_t *blocks, const int32_t *counts, const void *workspace,
                           size_t ws_bytes);
int h3_check_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                              const uint16_t *v, int64_t ld_v, const uint16_t *o, int64_t ld_o,
                              int64_t L_buf, int64_t valid_len, int64_t prefix_len, int32_t heads,
                              int32_t head_dim, float softmax_scale, const uint16_t *blocks,
                              const int32_t *counts, const void *workspace, size_t ws_bytes);

int h3_check_mxfp8_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K,
                            const uint8_t *q, int64_t ld_q, const uint8_t *scales);
int h3_check_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                          const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias,
                          const uint16_t *c, int64_t ldc, int64_t M_buf, int64_t M_valid, int64_t N, int64_t K,
                          int32_t epilogue, const uint16_t *resid, int64_t ld_r, const float *gate,
                          int64_t ld_gate_group, int32_t n_mod_groups);

int h3_check_fused_modulate_norm_mxfp8(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                       const float *shift, const float *scale, const float *gate,
                                       int64_t ld_mod_group, int32_t n_mod_groups, const uint16_t *x1_out,
                                       int64_t ld_x1, const uint8_t *hq, int64_t ld_hq, const uint8_t *hs,
                                       int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                       int32_t norm_type);
int h3_check_block_forward_mxfp8(const h3_dims *dims, const h3_block_weights_mxfp8 *w,
                                 const uint16_t *x, const uint16_t *y,
                                 const float *mod, int32_t n_mod_groups, const int32_t *mod_idx,
                                 const int32_t *pos, int64_t L_buf, int64_t valid_len,
                                 int64_t prefix_len, float tau,
                                 const void *workspace, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * h3_mfma_ceiling - a measured ceiling for the matrix-core roofline (not a
 * step of the block; a measurement aid for the GEMM and attention kernels).
 * Runs one workgroup of 4 waves per CU, each wave issuing `iters` rounds of
 * 16 MFMAs in the GEMM tile's register pattern (4 A and 4 B operands, 16
 * accumulators) on operands with varying bits, with no memory traffic; time
 * it on `stream` to get the sustained MFMA rate.
 *   dtype        H3_CEIL_BF16: v_mfma_f32_32x32x16_bf16;
 *                H3_CEIL_FP8: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3
 *                operands with unit E8M0 scales (the MXFP8 GEMM's MFMA).
 *                Other values: H3_ERR_UNSUPPORTED.
 *   iters        1 .. 2^20 rounds per wave.
 *   sink         device FP32 buffer of sink_floats >= 256 * (CU count)
 *                floats (4-byte aligned); receives one sum per thread so the
 *                products stay live. Its contents are not meaningful.
 *   flops        host double: set to the launch's MFMA flops.
 * H3_ERR_SHAPE when sink_floats is below 256 per CU of the current device.
 * ------------------------------------------------------------------------- */
enum { H3_CEIL_BF16 = 0, H3_CEIL_FP8 = 1 };
int h3_mfma_ceiling(int32_t dtype, int32_t iters, float *sink, int64_t sink_floats, double *flops, void *stream);
int h3_check_mfma_ceiling(int32_t dtype, int32_t iters, const float *sink, int64_t sink_floats,
                          const double *flops);

/* Human-readable name of a status code (static string). */
const char *h3_status_string(int status);
/* H3_ABI_VERSION of the built library. */
int h3_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* H3BLOCK_H */
