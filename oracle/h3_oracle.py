"""Plain FP64 CPU oracle of one MiniMax-H3 DiT block forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path never calls it, and it
shares no code with the HIP library or its Python binding.

Every function is the plain definition written out in float64 with numpy. There is
no blocking, fusion or reordering beyond what the definition states; library
primitives (matrix products, exp) serve as steps.

Sources (cited by page title and section):

* [Sol-H3] "Sol-H3: Recursive Self-Improvement for MiniMax-H3 Inference
  Acceleration on Sol-Engine across Cloud and Edge".
  - §3.5 "Kernel Fusion": the block's three operator groups: (1) residual
    addition with indexed gating, RMSNorm and indexed scale/shift modulation;
    (2) QK normalization with partial RoPE; (3) SwiGLU splitting, SiLU and
    multiplication. Hidden width 5376.
  - §3.5 "Precision-preserving LoRA fusion": BF16 rounding points (the SwiGLU
    gate product is kept in BF16 before the down projection).
  - §3.2 "Optimized attention collectives": packed QKV storage; flat
    (total, heads, head_dim) layout.
  - §3.2 "Quantized communication": a token/head record holds 3x128 QKV values,
    so the head width is 128.
  - §3.4 "Safety rails": sequence packing [text | conditioning video | audio |
    target video].
  - §3.3 "Compute Quantization" ("MXFP8 GEMM computation"): E4M3 values with one E8M0 scale per 32
    values along the reduction dimension, written by the producers.
  - §3.4 "Sparse Attention": Sol-Attn block selection by the threshold
    mu + tau * sigma per query block; prefix queries dense; prefix keys always
    attended.
* [vLLM-Omni H3] "MiniMax H3 on vLLM-Omni: integrating FastVideo FastH3" (blog).
  - §3.1: 58,758 valid tokens in a 58,816-token aligned buffer; the attention
    backend receives the valid length and drops the structural padding suffix.
  - §3.2: fused Q/K RMSNorm + RoPE; merged FP32 modulation, normalization and
    residual; fused SwiGLU.
* [SolarWM] "SolarWM H3 Realtime Interaction".
  - stage 2 "attention backend": queries are grouped (condition, audio,
    current video); video queries also read a longer history context.
  - stage 3 "history K/V reuse": the history K/V is concatenated once per
    refresh and reused by the chunk's four denoise forwards.

Readings where the pages are silent (each also listed in the design notes):
  R1 norm inside AdaLN is RMSNorm without an affine weight; LayerNorm optional.
  R3 eps = 1e-6 for every norm unless given.
  R4 modulation h = n * (1 + scale) + shift; gated residual x + gate * branch.
  R5 table rows (shift_a, scale_a, gate_a, shift_f, scale_f, gate_f).
  R7 QK-norm is per head over its 128 channels with one gain vector for q and
     one for k, shared by all heads.
  R8 partial RoPE rotates the first rot_dim channels of a head; default
     rotate-half pairing (i, i + rot_dim/2); omega_i = theta^(-2i/rot_dim);
     the angle is position * omega_i; position defaults to the packed row.
  R9 RMSNorm first, then RoPE.
  R10 attention is non-causal with scale 1/sqrt(head_dim); keys limited to
      the valid prefix [0, valid_len); padding query rows give 0.
  R11 w_qkv rows are q | k | v, each head-major; w_up rows are gate | up.
  R13 the exact result keeps no intermediate rounding (float64 throughout);
      an optional diagnosis mode rounds at the BF16 store points.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

# Row order of one modulation-table entry (reading R5).
SHIFT_A, SCALE_A, GATE_A, SHIFT_F, SCALE_F, GATE_F = range(6)


# ----------------------------------------------------------------------------
# Decoding of the bytes the GPU receives (storage formats, not the method).
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns (uint16) as float64.

    A BF16 number is the upper half of an IEEE binary32 number, so shifting the
    pattern into the high 16 bits of a 32-bit word gives the same value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(F64)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 value, ties to even (used only
    by the optional BF16-store-point diagnosis mode, reading R13).

    Rounding is done in two exact steps: float64 -> nearest binary32 would
    double-round, so the BF16 grid is computed directly from the float64 value:
    the spacing of BF16 at |a| is 2^(e - 7) for a in [2^e, 2^(e+1))."""
    a = np.asarray(a, dtype=F64)
    out = np.zeros_like(a)
    nz = (a != 0) & np.isfinite(a)
    m, e = np.frexp(a[nz])            # a = m * 2^e, 0.5 <= |m| < 1
    # BF16 has 8 significant bits: scale the mantissa to [128, 256).
    scaled = m * 256.0
    r = np.round(scaled)              # numpy rounds half to even
    out[nz] = np.ldexp(r, e - 8)
    out[~nz] = a[~nz]
    return out


# ----------------------------------------------------------------------------
# Normalisation and modulation (Sol-H3 §3.5 group (1); vLLM-Omni H3 §3.2).
# ----------------------------------------------------------------------------
def rms_norm(z: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis without affine weight: z / sqrt(mean(z^2) + eps)."""
    z = np.asarray(z, dtype=F64)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return z / np.sqrt(ms + eps)


def layer_norm(z: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis without affine weight: (z - mean) / sqrt(var + eps),
    with the population variance (optional norm type, reading R1)."""
    z = np.asarray(z, dtype=F64)
    mu = np.mean(z, axis=-1, keepdims=True)
    d = z - mu
    var = np.mean(d * d, axis=-1, keepdims=True)
    return d / np.sqrt(var + eps)


def modulate(n: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """AdaLN scale/shift modulation n * (1 + scale) + shift (reading R4)."""
    return n * (1.0 + scale) + shift


def modulate_norm(x, shift, scale, eps, norm_type=0):
    """Group (1) second half: normalise each row, then indexed scale/shift.

    `shift` and `scale` are per-row already (the caller gathers the table entry
    each row's index selects)."""
    n = rms_norm(x, eps) if norm_type == 0 else layer_norm(x, eps)
    return modulate(n, shift, scale)


def gated_residual(x, gate, branch):
    """Group (1) first half: residual addition with (indexed) gating x + gate * branch."""
    return x + gate * branch


# ----------------------------------------------------------------------------
# Precision-preserving LoRA consumer fusion (Sol-H3 report, §3.5 "Precision-
# preserving LoRA fusion"; Appendix B "Implementation scope"). The base
# projection and the LoRA branch each produce a BF16 output; the consumer uses
# their sum rounded to BF16 (never the unrounded sum, never merged weights).
# The final FFN consumer also keeps the gate product in BF16.
# ----------------------------------------------------------------------------
def lora_input(base, delta):
    """bf16(base + delta): the exact sum of the two BF16 branch outputs,
    rounded once to the nearest BF16 value, ties to even."""
    return round_to_bf16(np.asarray(base, dtype=F64) + np.asarray(delta, dtype=F64))


def gated_residual_bf16_product(x, gate, branch):
    """The final FFN consumer's residual: x + bf16(gate * branch), the gate
    product rounded to BF16 before the addition."""
    return np.asarray(x, dtype=F64) + round_to_bf16(np.asarray(gate, dtype=F64) * np.asarray(branch, dtype=F64))


def gather_mod(mod: np.ndarray, mod_idx, n_rows: int) -> np.ndarray:
    """Per-row modulation rows: entry mod_idx[r] of the [G, 6, H] table, or
    entry 0 for every row when no index is given (broadcast, reading R6).
    An index outside [0, G) selects the nearest end of the table (entry 0 or
    entry G - 1): the interface's rule for out-of-range indices, which the
    pages leave open (reading R5).
    Returns [n_rows, 6, H] float64."""
    mod = np.asarray(mod, dtype=F64)
    if mod_idx is None:
        return np.broadcast_to(mod[0], (n_rows,) + mod.shape[1:])
    idx = np.clip(np.asarray(mod_idx[:n_rows], dtype=np.int64), 0, mod.shape[0] - 1)
    return mod[idx]


# ----------------------------------------------------------------------------
# Linear layers (packed QKV: Sol-H3 §3.2; output and FFN projections).
# ----------------------------------------------------------------------------
def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """y = x W^T (+ b) with W stored [out, in]."""
    y = np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T
    if b is not None:
        y = y + np.asarray(b, dtype=F64)
    return y


# ----------------------------------------------------------------------------
# Group (2): QK RMSNorm with partial RoPE (Sol-H3 §3.5; vLLM-Omni H3 §3.2).
# ----------------------------------------------------------------------------
def head_rms_norm(t: np.ndarray, heads: int, head_dim: int, gain, eps: float) -> np.ndarray:
    """Per-head RMSNorm over the head's channels, times a per-channel gain shared
    by all heads (reading R7). t is [L, heads*head_dim]."""
    L = t.shape[0]
    th = np.asarray(t, dtype=F64).reshape(L, heads, head_dim)
    out = rms_norm(th, eps) * np.asarray(gain, dtype=F64)[None, None, :]
    return out.reshape(L, heads * head_dim)


def rope_frequencies(rot_dim: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/rot_dim) for i in [0, rot_dim/2) (reading R8)."""
    i = np.arange(rot_dim // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * i / rot_dim)


def apply_rope(t: np.ndarray, pos, heads: int, head_dim: int, rot_dim: int,
               theta: float, pairing: int = 0) -> np.ndarray:
    """Partial rotary embedding of each head's first rot_dim channels.

    pairing 0 (rotate-half): channel pair (i, i + rot_dim/2);
    pairing 1 (interleaved): channel pair (2i, 2i + 1).
    A pair (a, b) at angle phi = pos * omega_i becomes
    (a cos phi - b sin phi, a sin phi + b cos phi). Channels [rot_dim, head_dim)
    pass through. Rows with pos < 0 are left unrotated."""
    L = t.shape[0]
    out = np.array(t, dtype=F64).reshape(L, heads, head_dim)
    if rot_dim == 0:
        return out.reshape(L, heads * head_dim)
    pos = np.asarray(pos, dtype=F64)
    half = rot_dim // 2
    phi = pos[:, None] * rope_frequencies(rot_dim, theta)[None, :]   # [L, half]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    if pairing == 0:
        ia = np.arange(half)
        ib = ia + half
    else:
        ia = 2 * np.arange(half)
        ib = ia + 1
    a = out[:, :, ia].copy()
    b = out[:, :, ib].copy()
    ra = a * c - b * s
    rb = a * s + b * c
    keep = (pos < 0)
    ra[keep] = a[keep]
    rb[keep] = b[keep]
    out[:, :, ia] = ra
    out[:, :, ib] = rb
    return out.reshape(L, heads * head_dim)


def qk_norm_rope(t, pos, heads, head_dim, gain, eps, rot_dim, theta, pairing=0):
    """Group (2): RMSNorm per head (with gain), then partial RoPE (reading R9)."""
    return apply_rope(head_rms_norm(t, heads, head_dim, gain, eps), pos, heads,
                      head_dim, rot_dim, theta, pairing)


# ----------------------------------------------------------------------------
# Attention (Sol-H3 §3.2 profile; vLLM-Omni H3 §3.1 valid length;
# SolarWM stages 2-3 grouped queries and history K/V).
# ----------------------------------------------------------------------------
def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   q_chunk: int = 1024) -> np.ndarray:
    """softmax(q k^T * scale) v for one head over every key given.

    q [Lq, d], k and v [Lk, d]. The subtraction of the row maximum before exp is
    the usual exact rewriting of softmax. Queries are processed in chunks only to
    bound memory; each chunk is the full definition."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=F64)
    for a in range(0, q.shape[0], q_chunk):
        s = (q[a:a + q_chunk] @ k.T) * scale
        out[a:a + q_chunk] = _softmax_rows(s) @ v
    return out


def attention(q, k, v, heads: int, head_dim: int, scale=None, q_chunk: int = 1024):
    """Multi-head attention in the flat (rows, heads*head_dim) layout: each head
    attends over all rows of k/v given. Returns [Lq, heads*head_dim]."""
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(head_dim)
    Lq = q.shape[0]
    out = np.empty((Lq, heads * head_dim), dtype=F64)
    for h in range(heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        out[:, sl] = attention_head(q[:, sl], k[:, sl], v[:, sl], scale, q_chunk)
    return out


def attention_grouped(q, groups, heads: int, head_dim: int, n_rows: int, scale=None):
    """Grouped attention: each query group [q_begin, q_end) attends over the
    concatenation of its K/V segments (SolarWM stages 2-3). `groups` is a list of
    (q_begin, q_end, [(k_seg, v_seg), ...]). Rows outside every group give 0."""
    out = np.zeros((n_rows, heads * head_dim), dtype=F64)
    for (qb, qe, segs) in groups:
        if qe <= qb:
            continue
        kk = np.concatenate([np.asarray(s[0], dtype=F64) for s in segs], axis=0)
        vv = np.concatenate([np.asarray(s[1], dtype=F64) for s in segs], axis=0)
        out[qb:qe] = attention(q[qb:qe], kk, vv, heads, head_dim, scale)
    return out


# ----------------------------------------------------------------------------
# Sol-Attn block-sparse attention (Sol-H3 §3.4 "Sparse Attention").
#
# The sequence is [prefix | target video]; prefix = rows [0, prefix_len).
# Prefix queries attend densely over every valid key. Target queries are cut
# into query blocks of q_block rows counted from prefix_len, target keys into
# KV blocks of k_block rows counted from prefix_len (the last block of each may
# be short). For a query block, every target KV block gets a block-level score;
# the block is selected when its score exceeds mu + tau * sigma, mu and sigma
# being the mean and standard deviation of that query block's scores over all
# target KV blocks. The query block's rows attend exactly over the prefix keys
# (always-attended sinks) plus the keys of its selected blocks.
#
# Readings (the pages leave these open):
#   S1 block-level score = (mean of the block's q rows) . (mean of the KV
#      block's k rows) * scale, per head, before any softmax; q and k are the
#      attention inputs (after Q/K RMSNorm and RoPE).
#   S2 sigma is the population standard deviation (divide by the number of
#      target KV blocks); "exceed" is strict.
#   S3 block sizes: 256 query rows and 64 keys.
#   S4 the selection is an integer decision taken in FP32 (the kernel's
#      precision): pooled means, scores, mu, sigma and the threshold are FP32.
# ----------------------------------------------------------------------------
SPARSE_Q_BLOCK = 256
SPARSE_K_BLOCK = 64


def _blocks(n: int, size: int):
    return [(b, min(b + size, n)) for b in range(0, n, size)]


def sparse_block_scores(q, k, valid_len: int, prefix_len: int, heads: int, head_dim: int,
                        q_block: int = SPARSE_Q_BLOCK, k_block: int = SPARSE_K_BLOCK, scale=None):
    """Block-level attention scores of the target rows (reading S1), in FP32:
    returns [heads, n_qblocks, n_kblocks]."""
    f32 = np.float32
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(head_dim)
    P, V = int(prefix_len), int(valid_len)
    qb, kb = _blocks(V - P, q_block), _blocks(V - P, k_block)
    out = np.empty((heads, len(qb), len(kb)), dtype=f32)
    for h in range(heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        qt = np.asarray(q[P:V, sl], dtype=f32)
        kt = np.asarray(k[P:V, sl], dtype=f32)
        qbar = np.stack([qt[a:b].mean(axis=0, dtype=f32) for a, b in qb]) if qb else np.zeros((0, head_dim), f32)
        kbar = np.stack([kt[a:b].mean(axis=0, dtype=f32) for a, b in kb]) if kb else np.zeros((0, head_dim), f32)
        out[h] = (qbar @ kbar.T) * f32(scale)
    return out


def sparse_select(scores, tau: float):
    """Selection by the per-query-block threshold mu + tau * sigma (reading S2),
    in FP32. scores [..., n_kblocks]. Returns (selected bool mask, threshold)."""
    f32 = np.float32
    s = np.asarray(scores, dtype=f32)
    mu = s.mean(axis=-1, keepdims=True, dtype=f32)
    sigma = np.sqrt(np.square(s - mu).mean(axis=-1, keepdims=True, dtype=f32))
    thr = mu + f32(tau) * sigma
    return s > thr, thr[..., 0]


def sparse_attention(q, k, v, valid_len: int, prefix_len: int, heads: int, head_dim: int, selected,
                     q_block: int = SPARSE_Q_BLOCK, k_block: int = SPARSE_K_BLOCK, scale=None, n_rows=None):
    """Dense attention masked to the selected blocks (FP64). `selected`
    [heads, n_qblocks, n_kblocks] bool. Prefix rows attend over every valid
    key; a target query block over the prefix keys and its selected blocks.
    Rows past valid_len give 0."""
    P, V = int(prefix_len), int(valid_len)
    n_rows = V if n_rows is None else int(n_rows)
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(head_dim)
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    out = np.zeros((n_rows, heads * head_dim), dtype=F64)
    kb = _blocks(V - P, k_block)
    for h in range(heads):
        sl = slice(h * head_dim, (h + 1) * head_dim)
        if P > 0:
            out[:P, sl] = attention_head(q[:P, sl], k[:V, sl], v[:V, sl], scale)
        for bi, (a, b) in enumerate(_blocks(V - P, q_block)):
            keys = [np.arange(P)] + [np.arange(P + c, P + d) for j, (c, d) in enumerate(kb) if selected[h, bi, j]]
            idx = np.concatenate(keys).astype(np.int64)
            out[P + a:P + b, sl] = attention_head(q[P + a:P + b, sl], k[idx, sl], v[idx, sl], scale)
    return out


# ----------------------------------------------------------------------------
# MXFP8 (Sol-H3 §3.3 "Compute Quantization", "MXFP8 GEMM computation"): E4M3 values with one E8M0
# scale per 32 consecutive values along the reduction dimension.
#
# Readings (the pages name the formats, not the rule that picks a scale):
#   M1 E4M3 is the 8-bit float with 1 sign, 4 exponent (bias 7) and 3
#      mantissa bits, no infinities, one NaN pattern per sign (S.1111.111):
#      largest finite 448, smallest normal 2^-6, subnormal step 2^-9.
#      E8M0 is an unsigned biased exponent: code c stands for 2^(c - 127).
#   M2 the scale of a group of 32 is the microscaling rule: with amax the
#      group's largest magnitude, the shared exponent is floor(log2 amax)
#      minus 8 (the exponent of E4M3's largest binade), clamped to
#      [-127, 127]; a group of zeros takes the smallest scale, 2^-127.
#   M3 an element is v / 2^shared rounded to the nearest E4M3 value, ties to
#      the even code, with magnitudes above 448 saturating to 448.
#   M4 a GEMM on MXFP8 operands multiplies the scaled values exactly and
#      accumulates; the oracle dequantizes and multiplies in FP64.
#   M5 in the block, the quantizing producers quantize their exact outputs
#      (h, h2 from the norm, g from SwiGLU), with no BF16 step in between;
#      the attention output o is quantized from its BF16 value, since the
#      attention kernel returns BF16, and the residual stream x1 is taken at
#      its BF16 value (the block stores it in BF16) before the FFN-side norm
#      and residual. Quantization turns a last-bit difference of its input into
#      a whole E4M3 step, so these storage points are part of the definition.
# ----------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 bit patterns (uint8) -> float64 values (reading M1; NaN for the NaN patterns)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_round(v) -> np.ndarray:
    """Nearest E4M3 value of each real v, ties to even, saturating at +-448
    (reading M3). Returns float64 values (exactly representable in E4M3)."""
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    with np.errstate(divide='ignore'):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                       # below 2^-6 the step is fixed (subnormals)
    step = np.exp2(e - 3.0)
    q = np.round(a / step) * step                 # np.round: half to even
    q = np.minimum(q, E4M3_MAX)
    return np.sign(v) * q


def e4m3_encode(v) -> np.ndarray:
    """E4M3 bit patterns of values that are exactly representable (the output
    of e4m3_round); -0.0 and 0.0 both encode to 0x00 (sign of zero dropped)."""
    v = np.asarray(v, dtype=F64)
    table = e4m3_decode(np.arange(128))
    a = np.abs(v)
    idx = np.searchsorted(table[:127], a)
    assert np.all(table[np.minimum(idx, 126)] == a), "value not representable in E4M3"
    return (idx + np.where((v < 0) & (a > 0), 128, 0)).astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent of a group from its largest magnitude (reading M2)."""
    amax = np.asarray(amax, dtype=F64)
    with np.errstate(divide='ignore'):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0
    e = np.where(amax > 0, e, -127.0)
    return np.clip(e, -127.0, 127.0)


def mx_quantize(x, block: int = MX_BLOCK):
    """MXFP8 quantization of x [rows, K] along K in groups of 32 (K a multiple
    of 32). Returns (elements [rows, K] as float64 E4M3 values, shared
    exponents [rows, K/32] as float64 integers). The dequantized matrix is
    elements * 2^exponent, group by group."""
    x = np.asarray(x, dtype=F64)
    r, K = x.shape
    assert K % block == 0
    g = x.reshape(r, K // block, block)
    e = mx_scale_exponent(np.max(np.abs(g), axis=2))
    q = e4m3_round(g / np.exp2(e)[:, :, None])
    return q.reshape(r, K), e


def mx_dequantize(q, e, block: int = MX_BLOCK) -> np.ndarray:
    q = np.asarray(q, dtype=F64)
    r, K = q.shape
    return (q.reshape(r, K // block, block) * np.exp2(np.asarray(e, dtype=F64))[:, :, None]).reshape(r, K)


def linear_mxfp8(a_q, a_e, w_q, w_e, b=None) -> np.ndarray:
    """y = dequant(a) dequant(w)^T (+ b) in FP64 (reading M4)."""
    return linear(mx_dequantize(a_q, a_e), mx_dequantize(w_q, w_e), b)


# ----------------------------------------------------------------------------
# Group (3): SwiGLU (Sol-H3 §3.5; vLLM-Omni H3 §3.2).
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), written to avoid overflow for large |z|."""
    z = np.asarray(z, dtype=F64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu(u: np.ndarray, ffn: int) -> np.ndarray:
    """Split u = [gate | up] along columns, then silu(gate) * up (reading R11)."""
    u = np.asarray(u, dtype=F64)
    return silu(u[:, :ffn]) * u[:, ffn:2 * ffn]


# ----------------------------------------------------------------------------
# The whole block.
# ----------------------------------------------------------------------------
def block_forward(x, w, mod, *, heads: int, head_dim: int, ffn: int, valid_len: int,
                  rot_dim: int = 64, theta: float = 10000.0, eps: float = 1e-6,
                  norm_type: int = 0, pairing: int = 0, mod_idx=None, pos=None,
                  groups=None, scale=None, bf16_points: bool = False, sparse=None, mxfp8: bool = False):
    """One DiT block forward over a packed sequence of L_buf rows, valid_len valid.

    x      [L_buf, H] float64 (decoded BF16 values)
    w      dict with w_qkv [3H, H], w_o [H, H], w_up [2F, H], w_down [H, F],
           q_gain [head_dim], k_gain [head_dim], optional b_qkv, b_o, b_up, b_down
    mod    [G, 6, H] modulation table (reading R5 row order)
    groups None for dense attention over [0, valid_len); else a list of
           (q_begin, q_end, segs) where segs lists ('self', begin, len) for rows of
           this call's own K/V, or (k_array, v_array) for external (history) K/V.
    sparse None, or (prefix_len, tau): Sol-Attn block-sparse attention (Sol-H3
           §3.4) in place of dense attention, its blocks selected from this
           block's own q~ and k~; the selection is returned as 'sparse_sel'.
    mxfp8  the four projections on MXFP8 operands (Sol-H3 §3.3, readings
           M1-M5): the weights are quantized; h and h2 are quantized from the
           norm's exact values and g from the SwiGLU's (fused producers), o
           from its BF16 rounding (attention returns BF16). The dequantized
           operands are returned as h_q, o_q, h2_q and g_q.

    Steps (Sol-H3 §3.5 groups (1)-(3) around the projections):
      h   = modnorm(x; shift_a, scale_a)
      qkv = h W_qkv^T                     (q | k | v column blocks)
      q~, k~ = RoPE(RMSNorm_head(q) * g_q), RoPE(RMSNorm_head(k) * g_k)
      o   = attention(q~, k~, v)          (keys [0, valid_len) or per group)
      a   = o W_o^T ;   x1 = x + gate_a * a
      h2  = modnorm(x1; shift_f, scale_f)
      u   = h2 W_up^T ; g = silu(u_gate) * u_up
      f   = g W_down^T ; y = x1 + gate_f * f ;   y = 0 on padding rows
    Returns a dict with y and every intermediate, each [L_buf, .] with padding
    rows zero."""
    x = np.asarray(x, dtype=F64)
    L_buf, H = x.shape
    V = int(valid_len)
    rnd = round_to_bf16 if bf16_points else (lambda a: a)
    m = gather_mod(mod, mod_idx, V)
    xv = x[:V]
    if pos is None:
        posv = np.arange(V, dtype=F64)
    else:
        posv = np.asarray(pos[:V], dtype=F64)

    if mxfp8:
        wmx = {k_: mx_dequantize(*mx_quantize(w[k_])) for k_ in ('w_qkv', 'w_o', 'w_up', 'w_down')}
        mxq = lambda t: mx_dequantize(*mx_quantize(t))
    h_exact = modulate_norm(xv, m[:, SHIFT_A], m[:, SCALE_A], eps, norm_type)
    h = rnd(h_exact)
    extra = {}
    if mxfp8:
        extra['h_q'] = mxq(h_exact)
        qkv = rnd(linear(extra['h_q'], wmx['w_qkv'], w.get('b_qkv')))
    else:
        qkv = rnd(linear(h, w['w_qkv'], w.get('b_qkv')))
    q, k, v = qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:3 * H]
    qn = rnd(qk_norm_rope(q, posv, heads, head_dim, w['q_gain'], eps, rot_dim, theta, pairing))
    kn = rnd(qk_norm_rope(k, posv, heads, head_dim, w['k_gain'], eps, rot_dim, theta, pairing))
    sel = None
    if sparse is not None:
        P, tau = sparse
        sel, _ = sparse_select(sparse_block_scores(qn, kn, V, P, heads, head_dim), tau)
        o = sparse_attention(qn, kn, v, V, P, heads, head_dim, sel, scale=scale)
    elif groups is None:
        o = attention(qn, kn, v, heads, head_dim, scale)
    else:
        gl = []
        for (qb, qe, segs) in groups:
            ss = []
            for s in segs:
                if isinstance(s[0], str):
                    _, b0, ln = s
                    ss.append((kn[b0:b0 + ln], v[b0:b0 + ln]))
                else:
                    ss.append((s[0], s[1]))
            gl.append((qb, qe, ss))
        o = attention_grouped(qn, gl, heads, head_dim, V, scale)
    o = rnd(o)
    if mxfp8:
        extra['o_q'] = mxq(round_to_bf16(o))
        a = linear(extra['o_q'], wmx['w_o'], w.get('b_o'))
    else:
        a = linear(o, w['w_o'], w.get('b_o'))
    x1 = rnd(gated_residual(xv, m[:, GATE_A], a))
    if mxfp8:
        x1 = round_to_bf16(x1)
    h2_exact = modulate_norm(x1, m[:, SHIFT_F], m[:, SCALE_F], eps, norm_type)
    h2 = rnd(h2_exact)
    if mxfp8:
        extra['h2_q'] = mxq(h2_exact)
        u = linear(extra['h2_q'], wmx['w_up'], w.get('b_up'))
        g_exact = swiglu(u, ffn)
        g = rnd(g_exact)
        extra['g_q'] = mxq(g_exact)
        f = linear(extra['g_q'], wmx['w_down'], w.get('b_down'))
    else:
        u = linear(h2, w['w_up'], w.get('b_up'))
        g = rnd(swiglu(u, ffn))
        f = linear(g, w['w_down'], w.get('b_down'))
    y = rnd(gated_residual(x1, m[:, GATE_F], f))

    def pad(t):
        full = np.zeros((L_buf, t.shape[1]), dtype=F64)
        full[:V] = t
        return full

    out = {k_: pad(t_) for k_, t_ in dict(h=h, qkv=qkv, q=qn, k=kn, v=v, o=o, a=a,
                                           x1=x1, h2=h2, u=u, g=g, f=f, y=y, **extra).items()}
    if sel is not None:
        out['sparse_sel'] = sel
    return out


def block_forward_rows(x, w, mod, rows, *, heads: int, head_dim: int, ffn: int, valid_len: int,
                       rot_dim: int = 64, theta: float = 10000.0, eps: float = 1e-6, norm_type: int = 0,
                       pairing: int = 0, mod_idx=None, pos=None, groups=None, scale=None, q_chunk: int = 64,
                       mxfp8: bool = False):
    """block_forward restricted to the selected valid rows.

    Attention reads the keys and values of every valid row, so h, k~ and v are
    formed for all valid rows; every other step (q~, attention, the output
    projection, the FFN and the residuals) runs on the selected rows only. The
    definitions are those of block_forward, step for step, including its
    grouped attention (`groups` as in block_forward: a selected row attends
    over the segments of the group that contains it; a row outside every
    group gets o = 0). With mxfp8, the projections take MXFP8 operands at the
    quantization points of block_forward's mxfp8 option. Returns a dict of
    [len(rows), .] arrays."""
    x = np.asarray(x, dtype=F64)
    H = x.shape[1]
    V = int(valid_len)
    rows = np.asarray(rows, dtype=np.int64)
    m_all = gather_mod(mod, mod_idx, V)
    posv = np.arange(V, dtype=F64) if pos is None else np.asarray(pos[:V], dtype=F64)

    h_all = modulate_norm(x[:V], m_all[:, SHIFT_A], m_all[:, SCALE_A], eps, norm_type)
    w_qkv = np.asarray(w['w_qkv'], dtype=F64)
    if mxfp8:
        mxq = lambda t: mx_dequantize(*mx_quantize(t))
        w = dict(w)
        w_qkv = mxq(w_qkv)
        for k_ in ('w_o', 'w_up', 'w_down'):
            w[k_] = mxq(np.asarray(w[k_], dtype=F64))
        h_all = mxq(h_all)
    b_qkv = w.get('b_qkv')
    b = (lambda i: None) if b_qkv is None else (lambda i: np.asarray(b_qkv, dtype=F64)[i * H:(i + 1) * H])
    k_all = linear(h_all, w_qkv[H:2 * H], b(1))
    v_all = linear(h_all, w_qkv[2 * H:3 * H], b(2))
    kn = qk_norm_rope(k_all, posv, heads, head_dim, w['k_gain'], eps, rot_dim, theta, pairing)

    m = m_all[rows]
    h = h_all[rows]
    q = linear(h, w_qkv[:H], b(0))
    qn = qk_norm_rope(q, posv[rows], heads, head_dim, w['q_gain'], eps, rot_dim, theta, pairing)
    if groups is None:
        o = attention(qn, kn, v_all, heads, head_dim, scale, q_chunk)
    else:
        o = np.zeros((len(rows), H), dtype=F64)
        for (qb, qe, segs) in groups:
            sel = np.nonzero((rows >= qb) & (rows < qe))[0]
            if len(sel) == 0:
                continue
            ks, vs = [], []
            for sg in segs:
                if isinstance(sg[0], str):
                    _, b0, ln = sg
                    ks.append(kn[b0:b0 + ln])
                    vs.append(v_all[b0:b0 + ln])
                else:
                    ks.append(np.asarray(sg[0], dtype=F64))
                    vs.append(np.asarray(sg[1], dtype=F64))
            o[sel] = attention(qn[sel], np.concatenate(ks, axis=0), np.concatenate(vs, axis=0), heads, head_dim,
                               scale, q_chunk)
    a = linear(mxq(round_to_bf16(o)) if mxfp8 else o, w['w_o'], w.get('b_o'))
    x1 = gated_residual(x[rows], m[:, GATE_A], a)
    if mxfp8:
        x1 = round_to_bf16(x1)
    h2 = modulate_norm(x1, m[:, SHIFT_F], m[:, SCALE_F], eps, norm_type)
    u = linear(mxq(h2) if mxfp8 else h2, w['w_up'], w.get('b_up'))
    g = swiglu(u, ffn)
    f = linear(mxq(g) if mxfp8 else g, w['w_down'], w.get('b_down'))
    y = gated_residual(x1, m[:, GATE_F], f)
    return dict(h=h, q=qn, k=kn[rows], v=v_all[rows], o=o, a=a, x1=x1, h2=h2, g=g, f=f, y=y)
