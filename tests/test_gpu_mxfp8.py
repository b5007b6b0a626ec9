"""MXFP8 quantization and GEMMs (Sol-H3 report, §3.3 "Compute Quantization",
"MXFP8 GEMM computation") through the C ABI, against the oracle.

* Quantization: for BF16 inputs both sides scale exactly (a power of two) and
  round once to E4M3 in the same precision, so the codes must decode to the
  oracle's values exactly and the scale codes must be equal. Inputs include
  rounding ties, saturation (the top of a group's binade), E4M3-subnormal
  elements and all-zero groups.
* GEMM: operands given as MXFP8 (quantized by the oracle, or random codes and
  scales from the seeded generators), so both sides multiply the same values;
  the GPU output must match the oracle's dequantize-then-FP64 product to the
  parity bar (only FP32 accumulation order and the BF16 store differ).
"""
import numpy as np
import pytest
import torch

from oracle import h3_oracle as O
from video_diffusion_transformer_dit_amd import h3
from video_diffusion_transformer_dit_amd import inputs as I

from util import assert_parity, assert_zero_rows, dev_bf16, dev_f32, dev_i32, f64, poison

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def _scales_to_layout(e, rows):
    """Oracle shared exponents [rows, K/32] -> scale codes in the library's
    [K/128, rows, 4] layout (plain index bookkeeping)."""
    codes = (np.asarray(e, dtype=np.int64) + 127).astype(np.uint8)        # [rows, K/32]
    r, g = codes.shape
    return np.ascontiguousarray(codes.reshape(r, g // 4, 4).transpose(1, 0, 2))


def _scales_from_layout(s):
    """[K/128, rows, 4] -> [rows, K/32] shared exponents."""
    s = np.asarray(s, dtype=np.int64)
    kb, r, _ = s.shape
    return s.transpose(1, 0, 2).reshape(r, 4 * kb) - 127


def _mx_inputs_with_edges(name, rows, K):
    """BF16 test matrix: normal values at varied magnitudes, plus groups that
    hit rounding ties, saturation, E4M3-subnormal elements and zeros."""
    rng = I.rng_for(name)
    x = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-20, 20, size=(rows, 1)))
    g = K // 32
    for r in range(min(rows, 8)):
        base = np.exp2(float(rng.integers(-10, 10)))
        grp = slice(32 * (r % g), 32 * (r % g) + 32)
        if r % 4 == 0:      # ties: midpoints of E4M3 values (times the group scale 2^e with amax 256 * 2^e)
            v = np.array([1.0625, 1.1875, 2.125, 3.25, 0.5625, 17.0, 2 ** -7 * 1.5, 2 ** -9 * 0.5] * 4) * base
            v[0] = 256.0 * base
            x[r, grp] = v
        elif r % 4 == 1:    # saturation: amax in [448, 512) * 2^e
            x[r, grp] = rng.uniform(-500, 500, 32) * base
            x[r, 32 * (r % g)] = 505.0 * base
        elif r % 4 == 2:    # subnormal elements next to a large one
            x[r, grp] = rng.standard_normal(32) * 2.0 ** -14 * base
            x[r, 32 * (r % g)] = 300.0 * base
        else:
            x[r, grp] = 0.0
    return I.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("rows_buf,rows_valid,K", [(300, 291, 256), (70, 67, 5376), (8, 8, 128), (40, 0, 128)])
def test_mxfp8_quantize_matches_oracle(rows_buf, rows_valid, K):
    _say(f"mxfp8_quantize rows={rows_buf}/{rows_valid} K={K}")
    xb = _mx_inputs_with_edges(f"mxq.{rows_buf}.{K}", rows_buf, K)
    x = dev_bf16(xb)
    q = torch.full((rows_buf, K), 0x7F, dtype=torch.uint8, device="cuda")   # NaN codes: unwritten is visible
    s = torch.full(h3.mx_scales_shape(rows_buf, K), 0xEE, dtype=torch.uint8, device="cuda")
    h3.mxfp8_quantize(x, rows_valid, q, s)
    torch.cuda.synchronize()
    qc, sc = q.cpu().numpy(), s.cpu().numpy()
    if rows_valid:
        ref_q, ref_e = O.mx_quantize(O.bf16_to_f64(xb[:rows_valid]))
        np.testing.assert_array_equal(_scales_from_layout(sc)[:rows_valid], ref_e)
        np.testing.assert_array_equal(O.e4m3_decode(qc[:rows_valid]), ref_q)
    assert np.all(qc[rows_valid:] == 0) and np.all(_scales_from_layout(sc)[rows_valid:] == -127)


def _oracle_mx(name, rows, K, std=1.0):
    """An MXFP8 matrix made by the oracle from seeded BF16 values: (codes,
    exponents, dequantized values)."""
    xb = I.normal_bf16(name, (rows, K), std)
    qv, e = O.mx_quantize(O.bf16_to_f64(xb))
    return O.e4m3_encode(qv), e, O.mx_dequantize(qv, e)


@pytest.mark.parametrize("M_buf,M,N,K,epi", [(300, 291, 512, 256, h3.H3_EPI_STORE),
                                              (300, 291, 520, 384, h3.H3_EPI_STORE),
                                              (64, 64, 256, 128, h3.H3_EPI_STORE),
                                              (300, 280, 256, 512, h3.H3_EPI_RESIDUAL),
                                              (300, 291, 1024, 256, h3.H3_EPI_SWIGLU),
                                              (513, 513, 2080, 640, h3.H3_EPI_SWIGLU)])
def test_linear_mxfp8_matches_oracle(M_buf, M, N, K, epi):
    """Ragged M, N and K (odd stage counts), every epilogue, bias, indexed
    gates for the residual."""
    _say(f"linear_mxfp8 M={M_buf}/{M} N={N} K={K} epi={epi}")
    tag = f"{M_buf}.{N}.{K}.{epi}"
    ac, ae, ad = _oracle_mx(f"mxl.a.{tag}", M_buf, K)
    wc, we, wd = _oracle_mx(f"mxl.w.{tag}", N, K, 0.02)
    bias = I.normal_bf16(f"mxl.b.{tag}", (N,), 0.1)
    Nc = N // 2 if epi == h3.H3_EPI_SWIGLU else N
    c = poison((M_buf, Nc))
    kw = {}
    G = 3
    if epi == h3.H3_EPI_RESIDUAL:
        rb = I.normal_bf16(f"mxl.r.{tag}", (M_buf, N))
        gates = I.normal_f32(f"mxl.g.{tag}", (G, N), 0.3)
        idx = I.rng_for(f"mxl.i.{tag}").integers(0, G, size=M_buf).astype(np.int32)
        kw = dict(resid=dev_bf16(rb), gate=dev_f32(gates), ld_gate_group=N, n_mod_groups=G, mod_idx=dev_i32(idx))
    h3.linear_mxfp8(_u8(ac), _u8(_scales_to_layout(ae, M_buf)), _u8(wc), _u8(_scales_to_layout(we, N)), c, M, epi,
                    bias=dev_bf16(bias), **kw)
    torch.cuda.synchronize()
    z = O.linear(ad[:M], wd, O.bf16_to_f64(bias))
    if epi == h3.H3_EPI_SWIGLU:
        ref = O.swiglu(z, N // 2)
    elif epi == h3.H3_EPI_RESIDUAL:
        ref = O.gated_residual(O.bf16_to_f64(rb[:M]), gates[idx[:M]].astype(np.float64), z)
    else:
        ref = z
    assert_parity(f64(c)[:M], ref, "c", slack=2.0 ** -7 if epi == h3.H3_EPI_SWIGLU else 0.0)
    assert_zero_rows(c, M, "c")


def _random_mx(name, rows, K, lo=119, hi=127):
    """Seeded random MXFP8 operand: finite E4M3 codes and scale codes in
    [lo, hi] (generated inputs, not computed by either side)."""
    rng = I.rng_for(name)
    codes = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    e = rng.integers(lo, hi + 1, size=(rows, K // 32)) - 127
    return codes, e


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N,K,epi", [(3 * 5376, 5376, h3.H3_EPI_STORE), (2 * 21504, 5376, h3.H3_EPI_SWIGLU),
                                     (5376, 21504, h3.H3_EPI_RESIDUAL)])
def test_linear_mxfp8_full_size_sampled_rows(N, K, epi):
    """The block's projection shapes at 58,758 valid rows (58,816 buffer),
    sampled output rows against the oracle."""
    _say(f"linear_mxfp8 full size N={N} K={K} epi={epi}")
    M_buf, M = 58816, 58758
    tag = f"full.{N}.{K}"
    ac, ae = _random_mx(f"mxf.a.{tag}", M_buf, K, 116, 122)
    wc, we = _random_mx(f"mxf.w.{tag}", N, K, 110, 116)
    Nc = N // 2 if epi == h3.H3_EPI_SWIGLU else N
    c = torch.empty((M_buf, Nc), dtype=torch.bfloat16, device="cuda")
    kw = {}
    if epi == h3.H3_EPI_RESIDUAL:
        rb = I.normal_bf16(f"mxf.r.{tag}", (M_buf, N))
        gates = I.normal_f32(f"mxf.g.{tag}", (1, N), 0.3)
        kw = dict(resid=dev_bf16(rb), gate=dev_f32(gates), ld_gate_group=N)
    h3.linear_mxfp8(_u8(ac), _u8(_scales_to_layout(ae, M_buf)), _u8(wc), _u8(_scales_to_layout(we, N)), c, M, epi,
                    **kw)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([I.rng_for(f"mxf.rows.{tag}").choice(M, 24, replace=False), [0, 255, 256, M - 1]]))
    A = O.mx_dequantize(O.e4m3_decode(ac[rows]), ae[rows])
    W = O.mx_dequantize(O.e4m3_decode(wc), we)
    z = O.linear(A, W)
    if epi == h3.H3_EPI_SWIGLU:
        ref = O.swiglu(z, N // 2)
    elif epi == h3.H3_EPI_RESIDUAL:
        ref = O.gated_residual(O.bf16_to_f64(rb[rows]), gates[0].astype(np.float64), z)
    else:
        ref = z
    got = c[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    assert_parity(got, ref, "c", slack=2.0 ** -7 if epi == h3.H3_EPI_SWIGLU else 0.0)
    assert_zero_rows(c, M, "c")


def test_mxfp8_quantize_full_size_sampled_rows():
    """The quantizer at the block's activation shape (58,816 x 5,376, 58,758
    valid), sampled rows bit-exact against the oracle."""
    _say("mxfp8_quantize full size")
    M_buf, M, K = 58816, 58758, 5376
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202)
    x = (torch.randn((M_buf, K), generator=gen, device="cuda") * 3).to(torch.bfloat16)
    q = torch.empty((M_buf, K), dtype=torch.uint8, device="cuda")
    s = torch.empty(h3.mx_scales_shape(M_buf, K), dtype=torch.uint8, device="cuda")
    h3.mxfp8_quantize(x, M, q, s)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([I.rng_for("mxqf.rows").choice(M, 40, replace=False), [0, M - 1]]))
    rt = torch.from_numpy(rows).cuda()
    xs = x[rt].float().cpu().numpy().astype(np.float64)
    ref_q, ref_e = O.mx_quantize(xs)
    np.testing.assert_array_equal(O.e4m3_decode(q[rt].cpu().numpy()), ref_q)
    np.testing.assert_array_equal(_scales_from_layout(s[:, rt].cpu().numpy()), ref_e)
    assert torch.count_nonzero(q[M:]).item() == 0 and torch.count_nonzero(s[:, M:]).item() == 0
