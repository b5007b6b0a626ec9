// Host-side launch helpers and internal kernel launchers of libh3block.
#pragma once

#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

// H3_OK when the current device is gfx950 (cached per device).
int device_check();
// H3_OK when no launch error is pending, else H3_ERR_HIP.
int launch_status();

// ---- internal launchers (arguments already validated) ----
void launch_modnorm(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                    const float *shift, const float *scale, const float *gate, int64_t ld_mod_group,
                    int32_t n_mod_groups, const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1,
                    uint16_t *h_out, int64_t ld_h, int64_t L_buf, int64_t valid_len, int32_t hidden,
                    float eps, int32_t norm_type, hipStream_t stream);
void launch_qk_norm_rope(uint16_t *q, uint16_t *k, int64_t ld, const uint16_t *q_gain,
                         const uint16_t *k_gain, const int32_t *pos, int64_t L_buf, int64_t valid_len,
                         int32_t heads, int32_t rot_dim, int32_t pairing, float theta, float eps,
                         hipStream_t stream);
void launch_swiglu(const uint16_t *u, int64_t ld_u, uint16_t *g, int64_t ld_g, int64_t L_buf,
                   int64_t valid_len, int32_t ffn, hipStream_t stream);
void launch_modnorm_mx(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b, const float *shift,
                       const float *scale, const float *gate, int64_t ld_mod_group, int32_t n_mod_groups,
                       const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1, uint8_t *hq, int64_t ld_hq,
                       uint8_t *hs, int64_t L_buf, int64_t valid_len, int32_t hidden, float eps, int32_t norm_type,
                       hipStream_t stream);
void launch_mx_quantize(const uint16_t *x, int64_t ld_x, int64_t rows_buf, int64_t rows_valid, int64_t K, uint8_t *q,
                        int64_t ld_q, uint8_t *scales, hipStream_t stream);
void launch_linear_mxfp8(const uint8_t *a, int64_t lda, const uint8_t *a_scales, int64_t a_scale_rows,
                         const uint8_t *w, int64_t ldw, const uint8_t *w_scales, const uint16_t *bias, uint16_t *c,
                         int64_t ldc, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                         const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
                         int32_t n_mod_groups, const int32_t *mod_idx, hipStream_t stream,
                         uint8_t *cq = nullptr, int64_t ld_cq = 0, uint8_t *cs = nullptr, int64_t cs_rows = 0);
void launch_mx_zero_rows(uint8_t *q, int64_t ld_q, int64_t K, uint8_t *scales, int64_t rows_buf, int64_t r0,
                         int64_t r1, hipStream_t stream);
// Zero rows [r0, r1) of a BF16 matrix with `cols` columns at row stride ld.
void launch_zero_rows(uint16_t *p, int64_t ld, int64_t cols, int64_t r0, int64_t r1, hipStream_t stream);
// Copy rows of a BF16 matrix (cols columns) between two row strides.
void launch_copy_rows(const uint16_t *src, int64_t ld_src, uint16_t *dst, int64_t ld_dst, int64_t rows,
                      int64_t cols, hipStream_t stream);

// workspace: NULL, or at least gemm_plan(...).part_bytes bytes for the
// stream-K tail's partial sums (then the tail is split when the plan says so).
void launch_linear(const uint16_t *a, int64_t lda, const uint16_t *w, int64_t ldw, const uint16_t *bias,
                   uint16_t *c, int64_t ldc, int64_t M_valid, int64_t N, int64_t K, int32_t epilogue,
                   const uint16_t *resid, int64_t ld_r, const float *gate, int64_t ld_gate_group,
                   int32_t n_mod_groups, const int32_t *mod_idx, hipStream_t stream, void *workspace = nullptr);

void launch_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k,
                      const uint16_t *v, int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf,
                      int64_t valid_len, int32_t heads, float softmax_scale, const h3_qgroup *groups,
                      int32_t n_groups, void *workspace, hipStream_t stream);

void launch_sparse_select(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, int64_t valid_len,
                          int64_t prefix_len, int32_t heads, float tau, uint16_t *blocks, int32_t *counts,
                          void *workspace, hipStream_t stream);
void launch_sparse_attention(const uint16_t *q, int64_t ld_q, const uint16_t *k, int64_t ld_k, const uint16_t *v,
                             int64_t ld_v, uint16_t *o, int64_t ld_o, int64_t L_buf, int64_t valid_len,
                             int64_t prefix_len, int32_t heads, float softmax_scale, const uint16_t *blocks,
                             const int32_t *counts, void *workspace, hipStream_t stream);

}  // namespace h3
