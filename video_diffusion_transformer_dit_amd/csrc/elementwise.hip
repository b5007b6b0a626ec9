// HBM-bound fused elementwise kernels of the H3 DiT block for gfx950:
//   * modulate-norm  - operator group (1) of the Sol-H3 report, §3.5 "Kernel
//     Fusion": residual addition with indexed gating, RMSNorm and indexed
//     scale/shift modulation (merged FP32 modulation + norm + residual in the
//     vLLM-Omni H3 blog, §3.2);
//   * QK-norm + RoPE - operator group (2): per-head RMSNorm and partial rotary
//     embedding, in place on the packed QKV buffer;
//   * SwiGLU         - operator group (3): split, SiLU, multiply.
// All use 128-bit coalesced loads and stores of BF16 rows, FP32 arithmetic and
// round-to-nearest-even BF16 stores. Row offsets are formed in 64 bits (the
// vflash notes, "choosing a memory strategy": widen large offsets before the
// multiply); in-row offsets stay 32-bit.
#include <algorithm>

#include "h3_device.h"
#include "h3_runtime.h"

namespace h3 {
namespace {

// ---------------------------------------------------------------------------
// modulate-norm: SPAN lanes own ROWS rows (SPAN 64: one wavefront, ROWS rows;
// SPAN 256: the whole workgroup, one row); lane i holds 16-byte chunks
// i, i+SPAN, ... of each row in registers (NCH chunks max), so x (and the
// branch) are read once and h (and x1) written once. Wide rows take a
// workgroup each: the row's loads then leave every wave at once instead of
// one wave issuing them chunk after chunk.
// ---------------------------------------------------------------------------
struct ModnormArgs {
    const uint16_t *x;
    const uint16_t *branch;
    const uint16_t *delta;  // LoRA delta of the branch (LORA kernels)
    const float *shift;
    const float *scale;
    const float *gate;
    const int32_t *mod_idx;
    uint16_t *x1;
    uint16_t *h;
    int64_t ld_x, ld_b, ld_x1, ld_h, ld_mod, ld_d;
    int32_t gate_bf16;      // LORA: round the gate product to BF16 before the residual add
    uint8_t *hq;            // MX: h as E4M3 codes [L_buf, hidden] at ld_hq ...
    uint8_t *hs;            // ... and E8M0 scales [hidden / 128][L_buf][4]
    int64_t ld_hq;
    int64_t L_buf, valid;
    int32_t hidden, n_groups;
    float eps;
};

// LoRA consumer input: bf16(base + delta), round to nearest even. The FP32
// sum of two BF16 values is exact or, when the exponents are far apart, within
// an FP32 ulp of a value nowhere near a BF16 tie, so this is the correctly
// rounded BF16 sum (Sol-H3 report, §3.5 "Precision-preserving LoRA fusion":
// the consumer rounds base + delta to BF16 before using it).
__device__ __forceinline__ uint4 lora_add8(const uint4 &base, const uint4 &delta) {
    float fb[8], fd[8];
    unpack8(base, fb);
    unpack8(delta, fd);
#pragma unroll
    for (int e = 0; e < 8; ++e) fb[e] += fd[e];
    return pack8(fb);
}

// Round an FP32 value to BF16 (nearest even) and back.
__device__ __forceinline__ float bf16_round(float v) { return (float)(__bf16)v; }

__device__ __forceinline__ void load_f8(const float *p, float f[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// MX: instead of BF16 h, write h as MXFP8 straight from its FP32 values (the
// fused quantizing producer of Sol-H3 report, §3.3 "MXFP8 GEMM computation").
// A 32-wide group is the 4 consecutive chunks of 4 consecutive lanes; the 4
// groups of a 128-wide scale slab are the chunks of 16 consecutive lanes.
// Row sum of the per-lane partial sums v[0..3], in one association for both
// spans, so that every instance gives the same bits: with SPAN 256, thread
// 64 w + l holds the chunks w * 64 + l + 256 i in v[0]; with SPAN 64, lane l
// holds the chunks l + 64 (4 i + w) in v[w]. Either way the result is
// (S_0 + S_1) + (S_2 + S_3), S_w the wave sum of the chunks with
// (c / 64) % 4 == w, each lane adding its chunks in increasing order.
// The sums of ROWS rows at once (SPAN 256: one pair of barriers for all of
// them; red holds 4 floats per row).
template <int SPAN, int ROWS>
__device__ __forceinline__ void row_sums(const float (&v)[ROWS][4], float *red, float (&out)[ROWS]) {
    if (SPAN == 64) {
#pragma unroll
        for (int p = 0; p < ROWS; ++p)
            out[p] = (wave_sum(v[p][0]) + wave_sum(v[p][1])) + (wave_sum(v[p][2]) + wave_sum(v[p][3]));
        return;
    }
    float w[ROWS];
#pragma unroll
    for (int p = 0; p < ROWS; ++p) w[p] = wave_sum(v[p][0]);
    __syncthreads();  // red may still be read by a previous sum
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int p = 0; p < ROWS; ++p) red[4 * p + (threadIdx.x >> 6)] = w[p];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < ROWS; ++p) out[p] = (red[4 * p] + red[4 * p + 1]) + (red[4 * p + 2] + red[4 * p + 3]);
}

template <int NCH, int ROWS, bool BRANCH, int NORM, bool LORA = false, bool MX = false, int SPAN = 64>
__global__ __launch_bounds__(256) void modnorm_kernel(ModnormArgs a) {
    __shared__ float red[4 * ROWS];
    const int lane = SPAN == 64 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;  // chunk lane within the row
    const int64_t r0 = SPAN == 64 ? ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * ROWS : (int64_t)blockIdx.x * ROWS;
    if (r0 >= a.L_buf) return;  // uniform over the row's lanes
    const int nch = a.hidden >> 3;

    uint4 xv[ROWS][NCH];
    int grp[ROWS];
    bool valid[ROWS], inbuf[ROWS];
#pragma unroll
    for (int p = 0; p < ROWS; ++p) {
        const int64_t r = r0 + p;
        inbuf[p] = r < a.L_buf;
        valid[p] = r < a.valid;
        int g = 0;
        if (valid[p] && a.mod_idx) g = min(max(a.mod_idx[r], 0), a.n_groups - 1);
        grp[p] = g;
    }

    // Pass 1: load rows (forming x1 = x + gate * branch), accumulate the sum of
    // squares (RMSNorm) or the sum (LayerNorm).
    float acc[ROWS][4];
#pragma unroll
    for (int p = 0; p < ROWS; ++p)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[p][w] = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + SPAN * i;
        const int w = SPAN == 64 ? (i & 3) : 0;  // partial sum of the chunk (see row_sum)
        if (c < nch) {
            float gv[8];
            int gcur = -1;
#pragma unroll
            for (int p = 0; p < ROWS; ++p) {
                if (!valid[p]) continue;
                const int64_t r = r0 + p;
                uint4 xw = load_nt(a.x + r * a.ld_x + 8 * c);
                if (BRANCH) {
                    if (grp[p] != gcur) {
                        load_f8(a.gate + (int64_t)grp[p] * a.ld_mod + 8 * c, gv);
                        gcur = grp[p];
                    }
                    uint4 bw = load_nt(a.branch + r * a.ld_b + 8 * c);
                    if (LORA) bw = lora_add8(bw, *reinterpret_cast<const uint4 *>(a.delta + r * a.ld_d + 8 * c));
                    float xf[8], bf[8];
                    unpack8(xw, xf);
                    unpack8(bw, bf);
                    if (LORA && a.gate_bf16) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) xf[e] = xf[e] + bf16_round(gv[e] * bf[e]);
                    } else {
                        // one explicit FMA, so every instance of this kernel
                        // forms x1 identically (contraction is not left to the compiler)
#pragma unroll
                        for (int e = 0; e < 8; ++e) xf[e] = __builtin_fmaf(gv[e], bf[e], xf[e]);
                    }
                    xw = pack8(xf);
                    store_nt(a.x1 + r * a.ld_x1 + 8 * c, xw);
                }
                xv[p][i] = xw;
                float xf[8];
                unpack8(xw, xf);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[p][w] += NORM == 0 ? xf[e] * xf[e] : xf[e];
            }
        }
    }
    float mean[ROWS], inv[ROWS], sums[ROWS];
    row_sums<SPAN, ROWS>(acc, red, sums);
#pragma unroll
    for (int p = 0; p < ROWS; ++p) {
        const float s = sums[p];
        mean[p] = NORM == 0 ? 0.f : s / (float)a.hidden;
        if (NORM == 0) inv[p] = rsqrtf(s / (float)a.hidden + a.eps);
    }
    if (NORM == 1) {
        // two-pass population variance from the register copy
#pragma unroll
        for (int p = 0; p < ROWS; ++p)
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[p][w] = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + SPAN * i;
            const int w = SPAN == 64 ? (i & 3) : 0;
            if (c < nch) {
#pragma unroll
                for (int p = 0; p < ROWS; ++p) {
                    if (!valid[p]) continue;
                    float xf[8];
                    unpack8(xv[p][i], xf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float dlt = xf[e] - mean[p];
                        acc[p][w] += dlt * dlt;
                    }
                }
            }
        }
        row_sums<SPAN, ROWS>(acc, red, sums);
#pragma unroll
        for (int p = 0; p < ROWS; ++p) inv[p] = rsqrtf(sums[p] / (float)a.hidden + a.eps);
    }

    // Pass 2: h = n * (1 + scale) + shift; padding rows are written as zero.
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = lane + SPAN * i;
        if (c < nch) {
            float sh[8], sc[8];
            int gcur = -1;
#pragma unroll
            for (int p = 0; p < ROWS; ++p) {
                const int64_t r = r0 + p;
                if (!inbuf[p]) continue;
                if (!valid[p]) {
                    const uint4 z = make_uint4(0, 0, 0, 0);
                    if (MX) {
                        *reinterpret_cast<uint2 *>(a.hq + r * a.ld_hq + 8 * c) = make_uint2(0, 0);
                        if ((c & 15) == 0) *reinterpret_cast<uint32_t *>(a.hs + ((int64_t)(c >> 4) * a.L_buf + r) * 4) = 0;
                    } else if (!LORA || a.h) {
                        *reinterpret_cast<uint4 *>(a.h + r * a.ld_h + 8 * c) = z;
                    }
                    if (BRANCH) *reinterpret_cast<uint4 *>(a.x1 + r * a.ld_x1 + 8 * c) = z;
                    continue;
                }
                if (LORA && !a.h) continue;  // residual only
                if (grp[p] != gcur) {
                    load_f8(a.shift + (int64_t)grp[p] * a.ld_mod + 8 * c, sh);
                    load_f8(a.scale + (int64_t)grp[p] * a.ld_mod + 8 * c, sc);
                    gcur = grp[p];
                }
                float xf[8];
                unpack8(xv[p][i], xf);
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[e] = (xf[e] - mean[p]) * inv[p] * (1.f + sc[e]) + sh[e];
                if (MX) {
                    float amax = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xf[e]));
                    amax = fmaxf(amax, __shfl_xor(amax, 1));
                    amax = fmaxf(amax, __shfl_xor(amax, 2));
                    const int ex = mx_shared_exponent(amax);
                    const float is = mx_inv_scale(ex);
#pragma unroll
                    for (int e = 0; e < 8; ++e) xf[e] *= is;
                    *reinterpret_cast<uint2 *>(a.hq + r * a.ld_hq + 8 * c) = e4m3x8(xf);
                    const uint32_t code = (uint32_t)(ex + 127);
                    const uint32_t c1 = __shfl_down(code, 4), c2 = __shfl_down(code, 8), c3 = __shfl_down(code, 12);
                    if ((c & 15) == 0)
                        *reinterpret_cast<uint32_t *>(a.hs + ((int64_t)(c >> 4) * a.L_buf + r) * 4) =
                            code | (c1 << 8) | (c2 << 16) | (c3 << 24);
                } else {
                    store_nt(a.h + r * a.ld_h + 8 * c, pack8(xf));
                }
            }
        }
    }
}

template <int NCH, int SPAN = 64, int WG_ROWS = 1>
void modnorm_dispatch_nch(const ModnormArgs &a, bool branch, int norm, hipStream_t s, bool lora = false,
                          bool mx = false) {
    constexpr int ROWS = SPAN == 64 ? 2 : WG_ROWS;
    const int64_t waves = (a.L_buf + ROWS - 1) / ROWS;
    const dim3 grid((unsigned)(SPAN == 64 ? (waves + 3) / 4 : (a.L_buf + ROWS - 1) / ROWS));
    if (mx) {
        if (branch) {
            if (norm == 0) modnorm_kernel<NCH, ROWS, true, 0, false, true, SPAN><<<grid, 256, 0, s>>>(a);
            else modnorm_kernel<NCH, ROWS, true, 1, false, true, SPAN><<<grid, 256, 0, s>>>(a);
        } else {
            if (norm == 0) modnorm_kernel<NCH, ROWS, false, 0, false, true, SPAN><<<grid, 256, 0, s>>>(a);
            else modnorm_kernel<NCH, ROWS, false, 1, false, true, SPAN><<<grid, 256, 0, s>>>(a);
        }
    } else if (lora) {
        if (norm == 0) modnorm_kernel<NCH, ROWS, true, 0, true, false, SPAN><<<grid, 256, 0, s>>>(a);
        else modnorm_kernel<NCH, ROWS, true, 1, true, false, SPAN><<<grid, 256, 0, s>>>(a);
    } else if (branch) {
        if (norm == 0) modnorm_kernel<NCH, ROWS, true, 0, false, false, SPAN><<<grid, 256, 0, s>>>(a);
        else modnorm_kernel<NCH, ROWS, true, 1, false, false, SPAN><<<grid, 256, 0, s>>>(a);
    } else {
        if (norm == 0) modnorm_kernel<NCH, ROWS, false, 0, false, false, SPAN><<<grid, 256, 0, s>>>(a);
        else modnorm_kernel<NCH, ROWS, false, 1, false, false, SPAN><<<grid, 256, 0, s>>>(a);
    }
}

// Plain modulate-norm rows of 2,048 channels or more take a workgroup each
// (SPAN 256: 0.35 -> 0.29 ms at 58,758 x 5,376), two rows per workgroup for
// rows of 513-768 chunks (one pair of reductions and one read of the modulation
// vectors for both rows, loads of both in flight at once: 0.30 -> 0.26 ms,
// 0.24 ms with non-temporal loads and stores; four rows were slower);
// with the residual branch,
// which moves twice the bytes per row, two rows per wavefront (SPAN 64) stay
// faster (0.51 vs 0.58 ms), as do narrow rows. NCH covers the row's chunks.
void modnorm_dispatch(const ModnormArgs &a, bool branch, int norm, hipStream_t s, bool lora, bool mx) {
    const int nch = a.hidden / 8;
    if (!branch && nch >= 256) {
        const int need = (nch + 255) / 256;
        if (need <= 1) modnorm_dispatch_nch<1, 256>(a, branch, norm, s, lora, mx);
        else if (need <= 2) modnorm_dispatch_nch<2, 256>(a, branch, norm, s, lora, mx);
        else if (need <= 3) modnorm_dispatch_nch<3, 256, 2>(a, branch, norm, s, lora, mx);
        else if (need <= 4) modnorm_dispatch_nch<4, 256>(a, branch, norm, s, lora, mx);
        else modnorm_dispatch_nch<8, 256>(a, branch, norm, s, lora, mx);
    } else {
        const int need = (nch + 63) / 64;
        if (need <= 1) modnorm_dispatch_nch<1>(a, branch, norm, s, lora, mx);
        else if (need <= 2) modnorm_dispatch_nch<2>(a, branch, norm, s, lora, mx);
        else if (need <= 4) modnorm_dispatch_nch<4>(a, branch, norm, s, lora, mx);
        else if (need <= 8) modnorm_dispatch_nch<8>(a, branch, norm, s, lora, mx);
        else if (need <= 11) modnorm_dispatch_nch<11>(a, branch, norm, s, lora, mx);
        else if (need <= 16) modnorm_dispatch_nch<16>(a, branch, norm, s, lora, mx);
        else if (need <= 24) modnorm_dispatch_nch<24>(a, branch, norm, s, lora, mx);
        else modnorm_dispatch_nch<32>(a, branch, norm, s, lora, mx);
    }
}

// ---------------------------------------------------------------------------
// QK RMSNorm + partial RoPE: one workgroup per row; 16 lanes per 128-channel
// head vector (8 channels per lane); q heads then k heads.
// ---------------------------------------------------------------------------
struct QkArgs {
    uint16_t *q;
    uint16_t *k;
    uint16_t *v;                  // LORA: v column block, packed as bf16(v + dv) (may be null)
    const uint16_t *dq, *dk, *dv; // LORA deltas
    int64_t ld_d;
    const uint16_t *q_gain;
    const uint16_t *k_gain;
    const int32_t *pos;
    int64_t ld, L_buf, valid;
    int32_t heads, rot_dim, pairing;
    float theta, eps;
};

template <bool LORA = false>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(QkArgs a) {
    __shared__ float cs_cos[64];
    __shared__ float cs_sin[64];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const int slot = t >> 4;  // head-vector slot 0..15
    const int c = t & 15;     // 8-channel chunk within the head
    const int nhv = 2 * a.heads;
    if (r >= a.valid) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int hv = slot; hv < nhv; hv += 16) {
            uint16_t *base = hv < a.heads ? a.q + (int64_t)hv * 128 : a.k + (int64_t)(hv - a.heads) * 128;
            *reinterpret_cast<uint4 *>(base + r * a.ld + 8 * c) = z;
        }
        if (LORA && a.v)
            for (int cc = t; cc < a.heads * 16; cc += 256) *reinterpret_cast<uint4 *>(a.v + r * a.ld + 8 * cc) = z;
        return;
    }
    if (LORA && a.v)  // packing of v: bf16(v + dv)
        for (int cc = t; cc < a.heads * 16; cc += 256) {
            uint4 *pv = reinterpret_cast<uint4 *>(a.v + r * a.ld + 8 * cc);
            *pv = lora_add8(*pv, *reinterpret_cast<const uint4 *>(a.dv + r * a.ld_d + 8 * cc));
        }
    const int p = a.pos ? a.pos[r] : (int)r;
    const bool rot = p >= 0 && a.rot_dim > 0;
    const int half = a.rot_dim >> 1;
    if (rot && t < half) {
        // FP64 angle and its sine/cosine, rounded to FP32 (positions reach 6e4,
        // where an FP32 angle would carry errors of ~4e-3 rad).
        const double w = pow((double)a.theta, -2.0 * (double)t / (double)a.rot_dim);
        double sn, cn;
        sincos((double)p * w, &sn, &cn);
        cs_cos[t] = (float)cn;
        cs_sin[t] = (float)sn;
    }
    __syncthreads();
    float gq[8], gk[8];
    unpack8(*reinterpret_cast<const uint4 *>(a.q_gain + 8 * c), gq);
    unpack8(*reinterpret_cast<const uint4 *>(a.k_gain + 8 * c), gk);
    const int lane = t & 63;
    // rotate-half partner chunk (half is a multiple of 8)
    const int hc = half >> 3;
    int pc = c;
    if (c < hc) pc = c + hc;
    else if (c < 2 * hc) pc = c - hc;
    const int src_lane = (lane & ~15) | pc;
    const bool first_half = 8 * c < half;
    const bool rotated_chunk = 8 * c < a.rot_dim;

    for (int hv0 = 0; hv0 < nhv; hv0 += 16) {
        const int hv = hv0 + slot;
        const bool act = hv < nhv;
        const bool is_k = hv >= a.heads;
        uint16_t *ptr = nullptr;
        float f[8];
        if (act) {
            ptr = (is_k ? a.k + (int64_t)(hv - a.heads) * 128 : a.q + (int64_t)hv * 128) + r * a.ld + 8 * c;
            uint4 raw = load_nt(ptr);
            if (LORA) {
                const uint16_t *dp =
                    (is_k ? a.dk + (int64_t)(hv - a.heads) * 128 : a.dq + (int64_t)hv * 128) + r * a.ld_d + 8 * c;
                raw = lora_add8(raw, *reinterpret_cast<const uint4 *>(dp));
            }
            unpack8(raw, f);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = 0.f;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
        ss = sum16(ss);
        const float inv = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] * inv * (is_k ? gk[e] : gq[e]);
        if (rot) {
            if (a.pairing == 0) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = __shfl(f[e], src_lane);
                if (rotated_chunk) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = (8 * c + e) % half;
                        const float cs = cs_cos[j], sn = cs_sin[j];
                        // first half: a' = a cos - b sin; second half: b' = a sin + b cos
                        f[e] = first_half ? f[e] * cs - pv[e] * sn : pv[e] * sn + f[e] * cs;
                    }
                }
            } else if (rotated_chunk) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int j = (8 * c + e) >> 1;
                    const float cs = cs_cos[j], sn = cs_sin[j];
                    const float x0 = f[e], x1 = f[e + 1];
                    f[e] = x0 * cs - x1 * sn;
                    f[e + 1] = x0 * sn + x1 * cs;
                }
            }
        }
        if (act) store_nt(ptr, pack8(f));
    }
}

// ---------------------------------------------------------------------------
// SwiGLU: one thread per 8 output columns; a workgroup covers 2048 columns of
// one row.
// ---------------------------------------------------------------------------
template <bool LORA = false>
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t *u, int64_t ld_u, uint16_t *g,
                                                     int64_t ld_g, int64_t valid, int32_t ffn,
                                                     uint32_t blocks_per_row, const uint16_t *du = nullptr,
                                                     int64_t ld_du = 0) {
    const uint32_t row = blockIdx.x / blocks_per_row;
    const uint32_t cb = blockIdx.x - row * blocks_per_row;
    const int c = (int)(cb * 256 + threadIdx.x) * 8;
    if (c >= ffn) return;
    uint16_t *dst = g + (int64_t)row * ld_g + c;
    if ((int64_t)row >= valid) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(0, 0, 0, 0);
        return;
    }
    const uint16_t *src = u + (int64_t)row * ld_u + c;
    uint4 ua = load_nt(src), ub = load_nt(src + ffn);
    if (LORA) {
        const uint16_t *dsrc = du + (int64_t)row * ld_du + c;
        ua = lora_add8(ua, *reinterpret_cast<const uint4 *>(dsrc));
        ub = lora_add8(ub, *reinterpret_cast<const uint4 *>(dsrc + ffn));
    }
    float a[8], b[8];
    unpack8(ua, a);
    unpack8(ub, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = silu(a[e]) * b[e];
    store_nt(dst, pack8(a));
}

__global__ __launch_bounds__(256) void zero_rows_kernel(uint16_t *p, int64_t ld, int32_t chunks, int64_t r0,
                                                        int64_t rows) {
    const int64_t n = rows * chunks;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / chunks;
        const int c = (int)(i - r * chunks);
        *reinterpret_cast<uint4 *>(p + (r0 + r) * ld + 8 * c) = make_uint4(0, 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void copy_rows_kernel(const uint16_t *src, int64_t ld_s, uint16_t *dst,
                                                        int64_t ld_d, int32_t chunks, int64_t rows) {
    const int64_t n = rows * chunks;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / chunks;
        const int c = (int)(i - r * chunks);
        *reinterpret_cast<uint4 *>(dst + r * ld_d + 8 * c) =
            *reinterpret_cast<const uint4 *>(src + r * ld_s + 8 * c);
    }
}

}  // namespace

void launch_modnorm(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b, const float *shift,
                    const float *scale, const float *gate, int64_t ld_mod_group, int32_t n_mod_groups,
                    const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1, uint16_t *h_out, int64_t ld_h,
                    int64_t L_buf, int64_t valid_len, int32_t hidden, float eps, int32_t norm_type,
                    hipStream_t stream) {
    ModnormArgs a;
    a.x = x; a.branch = branch; a.shift = shift; a.scale = scale; a.gate = gate; a.mod_idx = mod_idx;
    a.x1 = x1_out; a.h = h_out;
    a.delta = nullptr; a.ld_d = 0; a.gate_bf16 = 0;
    a.ld_x = ld_x; a.ld_b = ld_b; a.ld_x1 = ld_x1; a.ld_h = ld_h;
    a.ld_mod = n_mod_groups > 1 ? ld_mod_group : 0;
    a.L_buf = L_buf; a.valid = valid_len; a.hidden = hidden; a.n_groups = n_mod_groups; a.eps = eps;
    const bool b = branch != nullptr;
    modnorm_dispatch(a, b, norm_type, stream, false, false);
}

void launch_qk_norm_rope(uint16_t *q, uint16_t *k, int64_t ld, const uint16_t *q_gain, const uint16_t *k_gain,
                         const int32_t *pos, int64_t L_buf, int64_t valid_len, int32_t heads, int32_t rot_dim,
                         int32_t pairing, float theta, float eps, hipStream_t stream) {
    QkArgs a;
    a.q = q; a.k = k; a.q_gain = q_gain; a.k_gain = k_gain; a.pos = pos;
    a.ld = ld; a.L_buf = L_buf; a.valid = valid_len;
    a.heads = heads; a.rot_dim = rot_dim; a.pairing = pairing; a.theta = theta; a.eps = eps;
    a.v = nullptr; a.dq = a.dk = a.dv = nullptr; a.ld_d = 0;
    qk_norm_rope_kernel<false><<<dim3((unsigned)L_buf), 256, 0, stream>>>(a);
}

void launch_swiglu(const uint16_t *u, int64_t ld_u, uint16_t *g, int64_t ld_g, int64_t L_buf, int64_t valid_len,
                   int32_t ffn, hipStream_t stream) {
    const uint32_t bpr = (uint32_t)((ffn / 8 + 255) / 256);
    swiglu_kernel<false><<<dim3((unsigned)(L_buf * bpr)), 256, 0, stream>>>(u, ld_u, g, ld_g, valid_len, ffn, bpr);
}

// Quantizing producer: h written as MXFP8 (codes hq at ld_hq, scales hs with
// L_buf scale rows) instead of BF16.
void launch_modnorm_mx(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b, const float *shift,
                       const float *scale, const float *gate, int64_t ld_mod_group, int32_t n_mod_groups,
                       const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1, uint8_t *hq, int64_t ld_hq,
                       uint8_t *hs, int64_t L_buf, int64_t valid_len, int32_t hidden, float eps, int32_t norm_type,
                       hipStream_t stream) {
    ModnormArgs a;
    a.x = x; a.branch = branch; a.shift = shift; a.scale = scale; a.gate = gate; a.mod_idx = mod_idx;
    a.x1 = x1_out; a.h = nullptr; a.hq = hq; a.hs = hs; a.ld_hq = ld_hq;
    a.delta = nullptr; a.ld_d = 0; a.gate_bf16 = 0;
    a.ld_x = ld_x; a.ld_b = ld_b; a.ld_x1 = ld_x1; a.ld_h = 0;
    a.ld_mod = n_mod_groups > 1 ? ld_mod_group : 0;
    a.L_buf = L_buf; a.valid = valid_len; a.hidden = hidden; a.n_groups = n_mod_groups; a.eps = eps;
    const bool b = branch != nullptr;
    modnorm_dispatch(a, b, norm_type, stream, false, true);
}

// LoRA consumer variants: the consumer rounds base + delta to BF16 first.
void launch_modnorm_lora(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                         const uint16_t *delta, int64_t ld_d, const float *shift, const float *scale,
                         const float *gate, int64_t ld_mod_group, int32_t n_mod_groups, const int32_t *mod_idx,
                         uint16_t *x1_out, int64_t ld_x1, uint16_t *h_out, int64_t ld_h, int64_t L_buf,
                         int64_t valid_len, int32_t hidden, float eps, int32_t norm_type, int32_t gate_bf16,
                         hipStream_t stream) {
    ModnormArgs a;
    a.x = x; a.branch = branch; a.shift = shift; a.scale = scale; a.gate = gate; a.mod_idx = mod_idx;
    a.x1 = x1_out; a.h = h_out;
    a.delta = delta; a.ld_d = ld_d; a.gate_bf16 = gate_bf16 ? 1 : 0;
    a.ld_x = ld_x; a.ld_b = ld_b; a.ld_x1 = ld_x1; a.ld_h = ld_h;
    a.ld_mod = n_mod_groups > 1 ? ld_mod_group : 0;
    a.L_buf = L_buf; a.valid = valid_len; a.hidden = hidden; a.n_groups = n_mod_groups; a.eps = eps;
    modnorm_dispatch(a, true, norm_type, stream, true, false);
}

void launch_qk_norm_rope_lora(uint16_t *q, uint16_t *k, uint16_t *v, int64_t ld, const uint16_t *dq,
                              const uint16_t *dk, const uint16_t *dv, int64_t ld_d, const uint16_t *q_gain,
                              const uint16_t *k_gain, const int32_t *pos, int64_t L_buf, int64_t valid_len,
                              int32_t heads, int32_t rot_dim, int32_t pairing, float theta, float eps,
                              hipStream_t stream) {
    QkArgs a;
    a.q = q; a.k = k; a.q_gain = q_gain; a.k_gain = k_gain; a.pos = pos;
    a.v = v; a.dq = dq; a.dk = dk; a.dv = dv; a.ld_d = ld_d;
    a.ld = ld; a.L_buf = L_buf; a.valid = valid_len;
    a.heads = heads; a.rot_dim = rot_dim; a.pairing = pairing; a.theta = theta; a.eps = eps;
    qk_norm_rope_kernel<true><<<dim3((unsigned)L_buf), 256, 0, stream>>>(a);
}

void launch_swiglu_lora(const uint16_t *u, int64_t ld_u, const uint16_t *du, int64_t ld_du, uint16_t *g,
                        int64_t ld_g, int64_t L_buf, int64_t valid_len, int32_t ffn, hipStream_t stream) {
    const uint32_t bpr = (uint32_t)((ffn / 8 + 255) / 256);
    swiglu_kernel<true><<<dim3((unsigned)(L_buf * bpr)), 256, 0, stream>>>(u, ld_u, g, ld_g, valid_len, ffn, bpr,
                                                                           du, ld_du);
}

void launch_zero_rows(uint16_t *p, int64_t ld, int64_t cols, int64_t r0, int64_t r1, hipStream_t stream) {
    if (r1 <= r0) return;
    const int64_t n = (r1 - r0) * (cols / 8);
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    zero_rows_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(p, ld, (int32_t)(cols / 8), r0, r1 - r0);
}

void launch_copy_rows(const uint16_t *src, int64_t ld_src, uint16_t *dst, int64_t ld_dst, int64_t rows,
                      int64_t cols, hipStream_t stream) {
    if (rows <= 0) return;
    const int64_t n = rows * (cols / 8);
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    copy_rows_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(src, ld_src, dst, ld_dst, (int32_t)(cols / 8),
                                                                rows);
}

}  // namespace h3

using namespace h3;

extern "C" {

int h3_fused_modulate_norm(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                           const float *shift, const float *scale, const float *gate, int64_t ld_mod_group,
                           int32_t n_mod_groups, const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1,
                           uint16_t *h_out, int64_t ld_h, int64_t L_buf, int64_t valid_len, int32_t hidden,
                           float eps, int32_t norm_type, void *stream) {
    int s = h3_check_fused_modulate_norm(x, ld_x, branch, ld_b, shift, scale, gate, ld_mod_group, n_mod_groups,
                                         x1_out, ld_x1, h_out, ld_h, L_buf, valid_len, hidden, eps, norm_type);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_modnorm(x, ld_x, branch, ld_b, shift, scale, gate, ld_mod_group, n_mod_groups, mod_idx, x1_out, ld_x1,
                   h_out, ld_h, L_buf, valid_len, hidden, eps, norm_type, (hipStream_t)stream);
    return launch_status();
}

int h3_qk_norm_rope(uint16_t *q, uint16_t *k, int64_t ld, const uint16_t *q_gain, const uint16_t *k_gain,
                    const int32_t *pos, int64_t L_buf, int64_t valid_len, int32_t heads, int32_t head_dim,
                    int32_t rot_dim, int32_t pairing, float theta, float eps, void *stream) {
    int s = h3_check_qk_norm_rope(q, k, ld, q_gain, k_gain, L_buf, valid_len, heads, head_dim, rot_dim, pairing,
                                  theta, eps);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_qk_norm_rope(q, k, ld, q_gain, k_gain, pos, L_buf, valid_len, heads, rot_dim, pairing, theta, eps,
                        (hipStream_t)stream);
    return launch_status();
}

int h3_swiglu(const uint16_t *u, int64_t ld_u, uint16_t *g, int64_t ld_g, int64_t L_buf, int64_t valid_len,
              int32_t ffn, void *stream) {
    int s = h3_check_swiglu(u, ld_u, g, ld_g, L_buf, valid_len, ffn);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_swiglu(u, ld_u, g, ld_g, L_buf, valid_len, ffn, (hipStream_t)stream);
    return launch_status();
}


int h3_fused_modulate_norm_lora(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                const uint16_t *delta, int64_t ld_d, const float *shift, const float *scale,
                                const float *gate, int64_t ld_mod_group, int32_t n_mod_groups,
                                const int32_t *mod_idx, uint16_t *x1_out, int64_t ld_x1, uint16_t *h_out,
                                int64_t ld_h, int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                int32_t norm_type, int32_t gate_bf16, void *stream) {
    int s = h3_check_fused_modulate_norm_lora(x, ld_x, branch, ld_b, delta, ld_d, shift, scale, gate, ld_mod_group,
                                              n_mod_groups, x1_out, ld_x1, h_out, ld_h, L_buf, valid_len, hidden,
                                              eps, norm_type, gate_bf16);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_modnorm_lora(x, ld_x, branch, ld_b, delta, ld_d, shift, scale, gate, ld_mod_group, n_mod_groups, mod_idx,
                        x1_out, ld_x1, h_out, ld_h, L_buf, valid_len, hidden, eps, norm_type, gate_bf16,
                        (hipStream_t)stream);
    return launch_status();
}

int h3_qk_norm_rope_lora(uint16_t *q, uint16_t *k, uint16_t *v, int64_t ld, const uint16_t *dq,
                         const uint16_t *dk, const uint16_t *dv, int64_t ld_d, const uint16_t *q_gain,
                         const uint16_t *k_gain, const int32_t *pos, int64_t L_buf, int64_t valid_len,
                         int32_t heads, int32_t head_dim, int32_t rot_dim, int32_t pairing, float theta, float eps,
                         void *stream) {
    int s = h3_check_qk_norm_rope_lora(q, k, v, ld, dq, dk, dv, ld_d, q_gain, k_gain, L_buf, valid_len, heads,
                                       head_dim, rot_dim, pairing, theta, eps);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_qk_norm_rope_lora(q, k, v, ld, dq, dk, dv, ld_d, q_gain, k_gain, pos, L_buf, valid_len, heads, rot_dim,
                             pairing, theta, eps, (hipStream_t)stream);
    return launch_status();
}

int h3_swiglu_lora(const uint16_t *u, int64_t ld_u, const uint16_t *du, int64_t ld_du, uint16_t *g,
                   int64_t ld_g, int64_t L_buf, int64_t valid_len, int32_t ffn, void *stream) {
    int s = h3_check_swiglu_lora(u, ld_u, du, ld_du, g, ld_g, L_buf, valid_len, ffn);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_swiglu_lora(u, ld_u, du, ld_du, g, ld_g, L_buf, valid_len, ffn, (hipStream_t)stream);
    return launch_status();
}

}  // extern "C"

extern "C" int h3_fused_modulate_norm_mxfp8(const uint16_t *x, int64_t ld_x, const uint16_t *branch, int64_t ld_b,
                                            const float *shift, const float *scale, const float *gate,
                                            int64_t ld_mod_group, int32_t n_mod_groups, const int32_t *mod_idx,
                                            uint16_t *x1_out, int64_t ld_x1, uint8_t *hq, int64_t ld_hq, uint8_t *hs,
                                            int64_t L_buf, int64_t valid_len, int32_t hidden, float eps,
                                            int32_t norm_type, void *stream) {
    int s = h3_check_fused_modulate_norm_mxfp8(x, ld_x, branch, ld_b, shift, scale, gate, ld_mod_group, n_mod_groups,
                                               x1_out, ld_x1, hq, ld_hq, hs, L_buf, valid_len, hidden, eps,
                                               norm_type);
    if (s != H3_OK || L_buf == 0) return s;
    if ((s = device_check()) != H3_OK) return s;
    launch_modnorm_mx(x, ld_x, branch, ld_b, shift, scale, gate, ld_mod_group, n_mod_groups, mod_idx, x1_out, ld_x1,
                      hq, ld_hq, hs, L_buf, valid_len, hidden, eps, norm_type, (hipStream_t)stream);
    return launch_status();
}
