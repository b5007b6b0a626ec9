"""Parity of each C-ABI entry point against the FP64 oracle on the same seeded
inputs, at sizes spanning several tiles with ragged tails, plus edge cases.
All calls go through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

from oracle import h3_oracle as O
from video_diffusion_transformer_dit_amd import h3
from video_diffusion_transformer_dit_amd import inputs as I

from util import (BF16_SLACK, assert_parity, assert_zero_rows, bits, dev_bf16, dev_f32, dev_i32, f64, poison)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# group (1): modulate-norm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,L,V", [(256, 512, 500), (5376, 130, 117), (1024, 1, 1), (512, 64, 0)])
@pytest.mark.parametrize("norm_type", [0, 1])
@pytest.mark.parametrize("with_branch", [False, True])
def test_modnorm(H, L, V, norm_type, with_branch):
    _say(f"modnorm H={H} L={L} V={V} norm={norm_type} branch={with_branch}")
    G = 3
    xb = I.normal_bf16("mn.x", (L, H))
    bb = I.normal_bf16("mn.b", (L, H))
    mod = I.normal_f32("mn.mod", (G, 6, H), 0.1)
    idx = I.rng_for("mn.idx").integers(0, G, size=L).astype(np.int32)
    x, br, md, ix = dev_bf16(xb), dev_bf16(bb), dev_f32(mod), dev_i32(idx)
    h_out = poison((L, H))
    x1_out = poison((L, H)) if with_branch else None
    h3.fused_modulate_norm(x, md[:, 0], md[:, 1], h_out, V, eps=1e-6, norm_type=norm_type,
                           branch=br if with_branch else None, gate=md[:, 2] if with_branch else None,
                           x1_out=x1_out, ld_mod_group=6 * H, n_mod_groups=G, mod_idx=ix)
    torch.cuda.synchronize()
    m = O.gather_mod(mod.astype(np.float64), idx, V)
    z = O.bf16_to_f64(xb[:V])
    if with_branch:
        z = O.gated_residual(z, m[:, O.GATE_A], O.bf16_to_f64(bb[:V]))
        if V:
            assert_parity(f64(x1_out)[:V], z, "x1")
        assert_zero_rows(x1_out, V, "x1")
    ref = O.modulate_norm(z, m[:, O.SHIFT_A], m[:, O.SCALE_A], 1e-6, norm_type)
    if V:
        assert_parity(f64(h_out)[:V], ref, "h")
    assert_zero_rows(h_out, V, "h")


def test_modnorm_gate_zero_is_bit_exact_and_inplace():
    H, L = 5376, 64
    _say("modnorm gate=0 in place")
    xb = I.normal_bf16("mz.x", (L, H))
    bb = I.normal_bf16("mz.b", (L, H), 100.0)
    mod = I.normal_f32("mz.mod", (1, 6, H), 0.1)
    mod[:, 2] = 0.0
    x, md = dev_bf16(xb), dev_f32(mod)
    h_out = poison((L, H))
    h3.fused_modulate_norm(x, md[:, 0], md[:, 1], h_out, L, branch=dev_bf16(bb), gate=md[:, 2], x1_out=x,
                           ld_mod_group=6 * H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(x), xb)


# ---------------------------------------------------------------------------
# group (2): QK RMSNorm + partial RoPE, in place on a packed qkv buffer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("heads,L,V", [(2, 512, 500), (42, 70, 67)])
@pytest.mark.parametrize("rot_dim,pairing", [(64, 0), (64, 1), (128, 0), (0, 0), (32, 0)])
@pytest.mark.parametrize("pos_kind", ["row", "explicit"])
def test_qk_norm_rope(heads, L, V, rot_dim, pairing, pos_kind):
    _say(f"qk_norm_rope heads={heads} L={L} V={V} rot={rot_dim} pairing={pairing} pos={pos_kind}")
    H = heads * 128
    qkv_b = I.normal_bf16("qk.qkv", (L, 3 * H), 3.0)
    gq = I.normal_bf16("qk.gq", (128,), 0.02, 1.0)
    gk = I.normal_bf16("qk.gk", (128,), 0.02, 1.0)
    if pos_kind == "row":
        pos = None
        posv = np.arange(L)
    else:
        posv = I.rng_for("qk.pos").integers(0, 60000, size=L).astype(np.int32)
        posv[::7] = -1     # rows with a negative position are not rotated
        pos = dev_i32(posv)
    qkv = dev_bf16(qkv_b)
    h3.qk_norm_rope(qkv[:, :H], qkv[:, H:2 * H], dev_bf16(gq), dev_bf16(gk), V, heads, rot_dim, pairing, 1e4,
                    1e-6, pos=pos)
    torch.cuda.synchronize()
    got = f64(qkv)
    src = O.bf16_to_f64(qkv_b)
    for name, sl, g in (("q", slice(0, H), gq), ("k", slice(H, 2 * H), gk)):
        ref = O.qk_norm_rope(src[:V, sl], posv[:V], heads, 128, O.bf16_to_f64(g), 1e-6, rot_dim, 1e4, pairing)
        assert_parity(got[:V, sl], ref, name)
        assert_zero_rows(qkv[:, sl], V, name)
    # v columns untouched, bit for bit
    np.testing.assert_array_equal(bits(qkv[:, 2 * H:]), qkv_b[:, 2 * H:])


# ---------------------------------------------------------------------------
# group (3): SwiGLU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F,L,V", [(1024, 512, 500), (21504, 20, 19), (8, 3, 3)])
def test_swiglu(F, L, V):
    _say(f"swiglu F={F} L={L} V={V}")
    ub = I.normal_bf16("sw.u", (L, 2 * F), 2.0)
    g = poison((L, F))
    h3.swiglu(dev_bf16(ub), g, V, F)
    torch.cuda.synchronize()
    ref = O.swiglu(O.bf16_to_f64(ub[:V]), F)
    assert_parity(f64(g)[:V], ref, "g", slack=BF16_SLACK)
    assert_zero_rows(g, V, "g")


def test_swiglu_full_size_beyond_2_31_elements():
    """The standalone SwiGLU call at the block's full FFN shape: u is
    [58,816 x 43,008] (2.53e9 elements, so element offsets pass 2^31 from row
    49,933 on) and g [58,816 x 21,504] (2.53 GB). Sampled rows, including the
    last 64 valid rows, against the oracle; every padding row +0.0 and no
    element left unwritten."""
    L, V, F = 58816, 58758, 21504
    _say(f"swiglu full size L={L} V={V} F={F}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260903)
    u = (torch.randn((L, 2 * F), generator=gen, device="cuda") * 2.0).to(torch.bfloat16)
    g = poison((L, F))
    h3.swiglu(u, g, V, F)
    torch.cuda.synchronize()
    assert not torch.isnan(g).any().item(), "g: unwritten (NaN) elements"
    pick = np.random.default_rng(7)
    rows = np.unique(np.concatenate([pick.choice(V, size=48, replace=False), np.arange(V - 64, V), [0]]))
    assert (rows.max() * 2 * F) >= 2 ** 31
    ur = O.bf16_to_f64(bits(u[torch.from_numpy(rows).cuda()]))
    ref = O.swiglu(ur, F)
    assert_parity(f64(g[torch.from_numpy(rows).cuda()]), ref, "g", slack=BF16_SLACK)
    assert_zero_rows(g, V, "g")


# ---------------------------------------------------------------------------
# projections (MFMA GEMM) with their epilogues
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,Mv,N,K", [(300, 291, 512, 256), (600, 599, 768, 5376), (64, 1, 256, 64),
                                      (257, 257, 264, 128), (130, 129, 256, 192)])
@pytest.mark.parametrize("bias", [False, True])
def test_linear_store(M, Mv, N, K, bias):
    _say(f"linear store M={M} Mv={Mv} N={N} K={K} bias={bias}")
    ab = I.normal_bf16("ln.a", (M, K))
    wb = I.normal_bf16("ln.w", (N, K), 0.02)
    bb = I.normal_bf16("ln.b", (N,), 0.5)
    c = poison((M, N))
    h3.linear(dev_bf16(ab), dev_bf16(wb), c, Mv, h3.H3_EPI_STORE, bias=dev_bf16(bb) if bias else None)
    torch.cuda.synchronize()
    ref = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb), O.bf16_to_f64(bb) if bias else None)
    assert_parity(f64(c)[:Mv], ref, "c")
    assert_zero_rows(c, Mv, "c")


@pytest.mark.parametrize("stages", list(range(1, 12)))
def test_linear_every_stage_count(stages):
    """K = 64 x 1..11: the main loop runs five K stages per iteration over a
    ring of five LDS operand tiles, then the remaining 0-4 stages each from its
    own ring position; every loop count and remainder against the oracle, on a
    ragged 2 x 2 tile grid."""
    M, Mv, N, K = 260, 258, 264, 64 * stages
    _say(f"linear stages={stages} M={M} Mv={Mv} N={N} K={K}")
    ab = I.normal_bf16(f"lst{stages}.a", (M, K))
    wb = I.normal_bf16(f"lst{stages}.w", (N, K), 0.05)
    c = poison((M, N))
    h3.linear(dev_bf16(ab), dev_bf16(wb), c, Mv, h3.H3_EPI_STORE)
    torch.cuda.synchronize()
    ref = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb), None)
    assert_parity(f64(c)[:Mv], ref, "c")
    assert_zero_rows(c, Mv, "c")


@pytest.mark.parametrize("M,Mv,N,K,G", [(300, 291, 512, 256, 1), (520, 515, 5376, 512, 3),
                                           (70, 66, 256, 320, 2)])
def test_linear_gated_residual(M, Mv, N, K, G):
    _say(f"linear residual M={M} N={N} K={K} G={G}")
    ab = I.normal_bf16("lr.a", (M, K))
    wb = I.normal_bf16("lr.w", (N, K), 0.05)
    rb = I.normal_bf16("lr.r", (M, N))
    mod = I.normal_f32("lr.mod", (G, 6, N), 0.5)
    idx = I.rng_for("lr.idx").integers(0, G, size=M).astype(np.int32)
    md = dev_f32(mod)
    c = poison((M, N))
    h3.linear(dev_bf16(ab), dev_bf16(wb), c, Mv, h3.H3_EPI_RESIDUAL, resid=dev_bf16(rb), gate=md[:, 2],
              ld_gate_group=6 * N, n_mod_groups=G, mod_idx=dev_i32(idx) if G > 1 else None)
    torch.cuda.synchronize()
    m = O.gather_mod(mod.astype(np.float64), idx if G > 1 else None, Mv)
    branch = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb))
    ref = O.gated_residual(O.bf16_to_f64(rb[:Mv]), m[:, O.GATE_A], branch)
    assert_parity(f64(c)[:Mv], ref, "x1")
    # The gated branch alone (the residual dominates the sum): its error, less
    # the BF16 rounding every store of x1 makes (at most half an ulp of x1, so
    # at most 2^-8 |x1|), is held to the standard bar against the branch.
    err = f64(c)[:Mv] - ref
    left = np.sign(err) * np.maximum(np.abs(err) - 2.0 ** -8 * np.abs(ref), 0.0)
    gb = ref - O.bf16_to_f64(rb[:Mv])
    assert_parity(gb + left, gb, "gate*branch less x1 rounding")
    assert_zero_rows(c, Mv, "x1")


def test_mod_idx_out_of_range_is_clamped():
    """Table indices outside [0, G) select the nearest end of the table (entry
    0 below, entry G - 1 above), as the interface states: in modulate-norm
    with and without the residual branch, and in the gated-residual GEMM
    epilogue."""
    G, H, L, V = 3, 512, 80, 77
    _say(f"mod_idx out of range G={G} H={H} L={L} V={V}")
    idx = I.rng_for("oor.idx").integers(0, G, size=L).astype(np.int32)
    idx[::5] = -1
    idx[1::7] = G
    idx[2::11] = np.iinfo(np.int32).max
    idx[3::13] = np.iinfo(np.int32).min
    idx[4::9] = 1000
    xb = I.normal_bf16("oor.x", (L, H))
    bb = I.normal_bf16("oor.b", (L, H))
    wb = I.normal_bf16("oor.w", (H, H), 0.05)
    mod = I.normal_f32("oor.mod", (G, 6, H), 0.5)
    md, ix = dev_f32(mod), dev_i32(idx)
    m = O.gather_mod(mod.astype(np.float64), idx, V)
    for with_branch in (False, True):
        h_out = poison((L, H))
        x1_out = poison((L, H)) if with_branch else None
        h3.fused_modulate_norm(dev_bf16(xb), md[:, 0], md[:, 1], h_out, V,
                               branch=dev_bf16(bb) if with_branch else None,
                               gate=md[:, 2] if with_branch else None, x1_out=x1_out, ld_mod_group=6 * H,
                               n_mod_groups=G, mod_idx=ix)
        torch.cuda.synchronize()
        z = O.bf16_to_f64(xb[:V])
        if with_branch:
            z = O.gated_residual(z, m[:, O.GATE_A], O.bf16_to_f64(bb[:V]))
            assert_parity(f64(x1_out)[:V], z, "x1 (modnorm)")
        assert_parity(f64(h_out)[:V], O.modulate_norm(z, m[:, O.SHIFT_A], m[:, O.SCALE_A], 1e-6), "h")
    c = poison((L, H))
    h3.linear(dev_bf16(xb), dev_bf16(wb), c, V, h3.H3_EPI_RESIDUAL, resid=dev_bf16(bb), gate=md[:, 2],
              ld_gate_group=6 * H, n_mod_groups=G, mod_idx=ix)
    torch.cuda.synchronize()
    ref = O.gated_residual(O.bf16_to_f64(bb[:V]), m[:, O.GATE_A],
                           O.linear(O.bf16_to_f64(xb[:V]), O.bf16_to_f64(wb)))
    assert_parity(f64(c)[:V], ref, "x1 (GEMM epilogue)")


@pytest.mark.parametrize("in_place", [False, True])
def test_linear_gated_residual_bias_ragged(in_place):
    """The residual epilogue with a bias, a ragged column tile (N = 264: the
    last tile's second wave has no valid column, its first wave 8) and ragged
    rows, indexed gates; also in place (c is the residual buffer, which the
    epilogue reads into LDS before it stores)."""
    M, Mv, N, K, G = 300, 291, 264, 128, 2
    _say(f"linear residual bias ragged in_place={in_place}")
    ab = I.normal_bf16("lrb.a", (M, K))
    wb = I.normal_bf16("lrb.w", (N, K), 0.05)
    bb = I.normal_bf16("lrb.b", (N,), 0.5)
    rb = I.normal_bf16("lrb.r", (M, N))
    mod = I.normal_f32("lrb.mod", (G, 6, N), 0.5)
    idx = I.rng_for("lrb.idx").integers(0, G, size=M).astype(np.int32)
    md = dev_f32(mod)
    r = dev_bf16(rb)
    c = r if in_place else poison((M, N))
    h3.linear(dev_bf16(ab), dev_bf16(wb), c, Mv, h3.H3_EPI_RESIDUAL, bias=dev_bf16(bb), resid=r, gate=md[:, 2],
              ld_gate_group=6 * N, n_mod_groups=G, mod_idx=dev_i32(idx))
    torch.cuda.synchronize()
    m = O.gather_mod(mod.astype(np.float64), idx, Mv)
    branch = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb), O.bf16_to_f64(bb))
    ref = O.gated_residual(O.bf16_to_f64(rb[:Mv]), m[:, O.GATE_A], branch)
    assert_parity(f64(c)[:Mv], ref, "x1")
    assert_zero_rows(c, Mv, "x1")


@pytest.mark.parametrize("M,Mv,F,K", [(300, 291, 512, 256), (260, 257, 1040, 512)])
@pytest.mark.parametrize("bias", [False, True])
def test_linear_swiglu(M, Mv, F, K, bias):
    _say(f"linear swiglu M={M} F={F} K={K} bias={bias}")
    ab = I.normal_bf16("lg.a", (M, K))
    wb = I.normal_bf16("lg.w", (2 * F, K), 0.05)
    bb = I.normal_bf16("lg.b", (2 * F,), 0.5)
    g = poison((M, F))
    h3.linear(dev_bf16(ab), dev_bf16(wb), g, Mv, h3.H3_EPI_SWIGLU, bias=dev_bf16(bb) if bias else None)
    torch.cuda.synchronize()
    u = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb), O.bf16_to_f64(bb) if bias else None)
    assert_parity(f64(g)[:Mv], O.swiglu(u, F), "g", slack=BF16_SLACK)
    assert_zero_rows(g, Mv, "g")


@pytest.mark.parametrize("epi,M,Mv,N,K", [(h3.H3_EPI_STORE, 1024, 1000, 2048, 7552),
                                          (h3.H3_EPI_RESIDUAL, 2700, 2600, 6144, 6656),
                                          (h3.H3_EPI_SWIGLU, 1024, 1000, 2048, 7552)])
def test_linear_stream_k_tail(epi, M, Mv, N, K):
    """Shapes whose last round of output tiles is split into K ranges
    (stream-K tail): 32 tiles of 118 stages cut into 256 ranges of 14-15
    stages (ranges straddle tiles), and 264 tiles = one whole round plus a
    tail of 8 tiles of 104 stages cut into 104 ranges of 8. Against the
    oracle, against the unsplit call (a different FP32 summation order
    only), and against a second call on the same workspace bit for bit (the
    fix-up adds the partial sums in K order)."""
    _say(f"linear stream-K epi={epi} M={M} Mv={Mv} N={N} K={K}")
    need = h3.linear_workspace_bytes(Mv, N, K, epi)
    assert need > 0, "the shape must take the split path"
    ab = I.normal_bf16("lk.a", (M, K))
    wb = I.normal_bf16("lk.w", (N, K), 0.05)
    bb = I.normal_bf16("lk.b", (N,), 0.5)
    cols = N // 2 if epi == h3.H3_EPI_SWIGLU else N
    kw = {"bias": dev_bf16(bb)}
    G = 3
    if epi == h3.H3_EPI_RESIDUAL:
        rb = I.normal_bf16("lk.r", (M, N))
        mod = I.normal_f32("lk.mod", (G, 6, N), 0.5)
        idx = I.rng_for("lk.idx").integers(0, G, size=M).astype(np.int32)
        md = dev_f32(mod)
        kw.update(resid=dev_bf16(rb), gate=md[:, 2], ld_gate_group=6 * N, n_mod_groups=G, mod_idx=dev_i32(idx))
    a, w = dev_bf16(ab), dev_bf16(wb)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    c = poison((M, cols))
    h3.linear(a, w, c, Mv, epi, workspace=ws, **kw)
    c2 = poison((M, cols))
    h3.linear(a, w, c2, Mv, epi, workspace=ws, **kw)
    c0 = poison((M, cols))
    h3.linear(a, w, c0, Mv, epi, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(c2), bits(c), err_msg="second split call differs")
    u = O.linear(O.bf16_to_f64(ab[:Mv]), O.bf16_to_f64(wb), O.bf16_to_f64(bb))
    if epi == h3.H3_EPI_STORE:
        ref, slack = u, 0.0
    elif epi == h3.H3_EPI_SWIGLU:
        ref, slack = O.swiglu(u, N // 2), BF16_SLACK
    else:
        m = O.gather_mod(mod.astype(np.float64), idx, Mv)
        ref, slack = O.gated_residual(O.bf16_to_f64(rb[:Mv]), m[:, O.GATE_A], u), 0.0
    assert_parity(f64(c)[:Mv], ref, "c (split tail)", slack=slack)
    assert_parity(f64(c)[:Mv], f64(c0)[:Mv], "c split vs unsplit", slack=slack)
    assert_zero_rows(c, Mv, "c")


@pytest.mark.parametrize("epi,Mv,N,K,split", [(h3.H3_EPI_RESIDUAL, 4096, 5376, 21504, True),
                                              (h3.H3_EPI_RESIDUAL, 4096, 5376, 5376, True),
                                              (h3.H3_EPI_STORE, 5424, 16128, 5376, False),
                                              (h3.H3_EPI_SWIGLU, 5424, 43008, 5376, False)])
def test_linear_block_shapes_full_size(epi, Mv, N, K, split):
    """The block's projections at full width, in the launches the block
    makes with its workspace: at 4,096 rows the down and output projections
    (336 tiles: one round plus a stream-K tail of 80 tiles in 256 ranges),
    at the streaming forward's 5,424 rows the QKV projection (1,386 tiles,
    no split) and up + SwiGLU (3,696 tiles, the last rounds drawn). Against
    the call without a workspace over every element (bit for bit where
    nothing is split, else the FP32 summation slack) and sampled rows, most
    of them in the last tile rows, against the oracle."""
    _say(f"linear full size epi={epi} Mv={Mv} N={N} K={K}")
    need = h3.linear_workspace_bytes(Mv, N, K, epi)
    assert (need > 256) == split
    ab = I.normal_bf16("lf.a", (Mv, K))
    wb = I.normal_bf16("lf.w", (N, K), 0.02)
    bb = I.normal_bf16("lf.b", (N,), 0.5)
    cols = N // 2 if epi == h3.H3_EPI_SWIGLU else N
    kw = {"bias": dev_bf16(bb)}
    if epi == h3.H3_EPI_RESIDUAL:
        rb = I.normal_bf16("lf.r", (Mv, N))
        mod = I.normal_f32("lf.mod", (1, 6, N), 0.5)
        kw.update(resid=dev_bf16(rb), gate=dev_f32(mod)[:, 2], n_mod_groups=1)
    a, w = dev_bf16(ab), dev_bf16(wb)
    ws = torch.full((max(need, 1),), 0x7F, dtype=torch.uint8, device="cuda") if need else None
    c = poison((Mv, cols))
    h3.linear(a, w, c, Mv, epi, workspace=ws, **kw)
    c0 = poison((Mv, cols))
    h3.linear(a, w, c0, Mv, epi, **kw)
    torch.cuda.synchronize()
    slack = BF16_SLACK if epi == h3.H3_EPI_SWIGLU else 0.0
    if split:
        assert_parity(f64(c), f64(c0), "c split vs unsplit", slack=slack)
    else:
        np.testing.assert_array_equal(bits(c), bits(c0), err_msg="workspace call differs")
    rows = np.unique(np.concatenate([np.arange(0, Mv, 613), np.arange(Mv - 512, Mv, 37), np.arange(Mv - 4, Mv)]))
    u = O.linear(O.bf16_to_f64(ab[rows]), O.bf16_to_f64(wb), O.bf16_to_f64(bb))
    if epi == h3.H3_EPI_SWIGLU:
        ref = O.swiglu(u, N // 2)
    elif epi == h3.H3_EPI_RESIDUAL:
        m = O.gather_mod(mod.astype(np.float64), None, Mv)[rows]
        ref = O.gated_residual(O.bf16_to_f64(rb[rows]), m[:, O.GATE_A], u)
    else:
        ref = u
    assert_parity(f64(c)[rows], ref, "c (sampled rows)", slack=slack)


@pytest.mark.parametrize("epi,Mv,N,K", [(h3.H3_EPI_STORE, 2000, 65536, 192), (h3.H3_EPI_SWIGLU, 1900, 65536, 128),
                                        (h3.H3_EPI_STORE, 2000, 65792, 3840)])
def test_linear_drawn_tiles(epi, Mv, N, K):
    """Launches of 8 rounds of output tiles or more: the last tiles of each
    XCD's range are drawn from counters in the workspace, by more workgroups
    than tiles. A tile's result does not depend on which workgroup computes
    it, so the output equals, bit for bit, the call without a workspace (every
    tile taken by workgroup index), also on a second call over the first
    call's counters; sampled rows (the last ones among them) against the
    oracle. 2,048 tiles (8 x 256, and 8 x 256 SwiGLU tiles of 128 columns),
    and 2,056 tiles of 60 stages whose last 8 are cut into stream-K ranges
    while the other 2,048 draw their last rounds (against the unsplit call
    with the FP32 summation slack)."""
    _say(f"linear drawn tiles epi={epi} Mv={Mv} N={N} K={K}")
    need = h3.linear_workspace_bytes(Mv, N, K, epi)
    split = need > 256
    assert need >= 256, "the shape must draw tiles"
    M = Mv + 5
    ab = I.normal_bf16("ld.a", (M, K))
    wb = I.normal_bf16("ld.w", (N, K), 0.05)
    bb = I.normal_bf16("ld.b", (N,), 0.5)
    cols = N // 2 if epi == h3.H3_EPI_SWIGLU else N
    a, w, b = dev_bf16(ab), dev_bf16(wb), dev_bf16(bb)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    c0 = poison((M, cols))
    h3.linear(a, w, c0, Mv, epi, bias=b)
    outs = []
    for _ in range(2):
        c = poison((M, cols))
        h3.linear(a, w, c, Mv, epi, bias=b, workspace=ws)
        outs.append(c)
    torch.cuda.synchronize()
    slack = BF16_SLACK if epi == h3.H3_EPI_SWIGLU else 0.0
    for i, c in enumerate(outs):
        if split:
            assert_parity(f64(c)[:Mv], f64(c0)[:Mv], f"c (call {i}) vs every tile by index", slack=slack)
        else:
            np.testing.assert_array_equal(bits(c), bits(c0), err_msg=f"call {i}: drawn tiles differ")
        assert_zero_rows(c, Mv, "c")
    np.testing.assert_array_equal(bits(outs[1]), bits(outs[0]), err_msg="second call differs")
    rows = np.unique(np.concatenate([np.arange(0, Mv, 97), np.arange(Mv - 8, Mv)]))
    u = O.linear(O.bf16_to_f64(ab[rows]), O.bf16_to_f64(wb), O.bf16_to_f64(bb))
    ref = O.swiglu(u, N // 2) if epi == h3.H3_EPI_SWIGLU else u
    assert_parity(f64(outs[0])[rows], ref, "c (sampled rows)", slack=slack)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _qkv(L, heads, tag, q_scale=1.0):
    H = heads * 128
    q = I.normal_bf16(f"{tag}.q", (L, H), q_scale)
    k = I.normal_bf16(f"{tag}.k", (L, H))
    v = I.normal_bf16(f"{tag}.v", (L, H))
    return q, k, v


@pytest.mark.parametrize("heads,L,V,q_scale", [(2, 512, 500, 1.0), (2, 512, 500, 8.0), (3, 700, 643, 1.0),
                                               (1, 70, 33, 3.0)])
@pytest.mark.parametrize("packed", [False, True])
def test_attention_dense(heads, L, V, q_scale, packed):
    _say(f"attention dense heads={heads} L={L} V={V} q_scale={q_scale} packed={packed}")
    H = heads * 128
    qb, kb, vb = _qkv(L, heads, "at", q_scale)
    if packed:
        qkv = dev_bf16(np.concatenate([qb, kb, vb], axis=1))
        q, k, v = qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:]
    else:
        q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = poison((L, H))
    h3.attention(q, k, v, o, V, heads)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(qb[:V]), O.bf16_to_f64(kb[:V]), O.bf16_to_f64(vb[:V]), heads, 128)
    assert_parity(f64(o)[:V], ref, "o")
    assert_zero_rows(o, V, "o")


@pytest.mark.parametrize("V", [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 255, 256, 257, 511, 513])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_attention_lengths_at_tile_boundaries(V, q_scale):
    """Valid lengths on both sides of every boundary the kernel has: 32-key
    half tiles, 64-key K/V tiles and 256-query workgroup tiles (the last tile
    of a length is partly masked, or exactly full), for the fixed-reference
    (q x 1) and the online (q x 8) form, in a buffer 7 rows longer."""
    heads, L = 2, V + 7
    _say(f"attention lengths heads={heads} L={L} V={V} q_scale={q_scale}")
    H = heads * 128
    qb, kb, vb = _qkv(L, heads, f"alen{V}", q_scale)
    o = poison((L, H))
    h3.attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, V, heads)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(qb[:V]), O.bf16_to_f64(kb[:V]), O.bf16_to_f64(vb[:V]), heads, 128)
    assert_parity(f64(o)[:V], ref, "o")
    if V == 1:  # one key: its value, bit for bit, on either form
        np.testing.assert_array_equal(bits(o[:1]), vb[:1])
    assert_zero_rows(o, V, "o")


def test_attention_fixed_and_online_workgroups_in_one_call():
    """Query tiles whose score bound |q| max|k| allows a fixed softmax
    reference and tiles whose bound does not (their q scaled by 8) in one
    call: the first are done by the fixed-reference kernel instance, the
    others by the online one; every row must match the oracle."""
    heads, L, V = 2, 1100, 1090
    H = heads * 128
    _say(f"attention fixed + online heads={heads} L={L} V={V}")
    qb, kb, vb = _qkv(L, heads, "amix")
    q = O.bf16_to_f64(qb)
    q[256:512] *= 8.0                       # query tile 1: bound far above the fixed range
    q[1000:1010] *= 8.0                     # a few rows of the last tile
    qb = I.f32_to_bf16_bits(q.astype(np.float32))
    o = poison((L, H))
    h3.attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, V, heads)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(qb[:V]), O.bf16_to_f64(kb[:V]), O.bf16_to_f64(vb[:V]), heads, 128)
    got = f64(o)
    # compared by kind of row (the max-error bar is relative to the slice's
    # RMS, and sharp rows, q x 8, have much larger outputs than soft ones)
    for a, b in ((0, 256), (256, 512), (512, 768), (768, 1000), (1000, 1010), (1010, 1024), (1024, V)):
        assert_parity(got[a:b], ref[a:b], f"o[{a}:{b}]")
    assert_zero_rows(o, V, "o")


def test_attention_long_launch_draws_items_and_defers_online_tiles():
    """A launch of 8 rounds of work items or more (42 heads x 49 query tiles =
    2,058 items): each XCD's last items are drawn from counters by surplus
    workgroups, and query tiles whose score bound rules out the fixed
    reference (their q scaled by 8; one of them among the drawn items at the
    end of the order) go to the online instance through the deferred-item
    list. Sampled rows of every kind against the oracle."""
    heads, V = 42, 12500
    L = V + 44
    H = heads * 128
    _say(f"attention long launch heads={heads} V={V}")
    q = O.bf16_to_f64(I.normal_bf16("along.q", (L, H)))
    sharp = [(256, 512), (6144, 6400), (12288, 12500)]   # query tiles 1, 24 and the last one
    for a, b in sharp:
        q[a:b] *= 8.0
    qb = I.f32_to_bf16_bits(q.astype(np.float32))
    kb = I.normal_bf16("along.k", (L, H))
    vb = I.normal_bf16("along.v", (L, H))
    kf = O.bf16_to_f64(kb[:V])
    for a, b in sharp:
        assert _score_bound(O.bf16_to_f64(qb[a:b]), kf) > 30.0
    for a in (0, 512, 6400, 12032):
        assert _score_bound(O.bf16_to_f64(qb[a:a + 256]), kf) <= 30.0
    o = poison((L, H))
    h3.attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, V, heads)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, V, 211), np.arange(256, 512, 37), np.arange(6144, 6400, 41),
                                     np.arange(V - 12, V)]))
    ref = O.attention(O.bf16_to_f64(qb[rows]), O.bf16_to_f64(kb[:V]), O.bf16_to_f64(vb[:V]), heads, 128)
    got = f64(o)[rows]
    is_sharp = np.zeros(len(rows), bool)
    for a, b in sharp:
        is_sharp |= (rows >= a) & (rows < b)
    assert is_sharp.sum() >= 10 and (~is_sharp).sum() >= 40
    assert_parity(got[is_sharp], ref[is_sharp], "o (online tiles)")
    assert_parity(got[~is_sharp], ref[~is_sharp], "o (fixed-reference tiles)")
    assert_zero_rows(o, V, "o")


def _rescale_count(q_rows, k_rows, slack=40.0):
    """Per (row, head): how often the online form must raise its softmax
    reference, restated from its rule: the reference starts at the row's
    largest scaled score among the first 32 keys, and each later 32-key half
    tile whose largest score exceeds the reference by more than the slack
    moves the reference up to that score."""
    c = np.log2(np.e) / np.sqrt(128.0)
    nq, nk = q_rows.shape[0], k_rows.shape[0]
    qh = q_rows.reshape(nq, -1, 128).transpose(1, 0, 2)
    kh = k_rows.reshape(nk, -1, 128).transpose(1, 0, 2)
    s = np.matmul(qh, kh.transpose(0, 2, 1)) * c          # [heads, nq, nk]
    halves = [s[:, :, i:i + 32].max(axis=-1) for i in range(0, nk, 32)]
    ref, count = halves[0], np.zeros(halves[0].shape, np.int64)
    for m in halves[1:]:
        up = m - ref > slack
        count += up
        ref = np.where(up, m, ref)
    return count


@pytest.mark.parametrize("pieces", [False, True])
def test_attention_online_rescales(pieces):
    """The online form's rescale path: keys whose norms ramp up 4x along the
    sequence (and a last stretch 12x), against peaked queries, so that each
    row's largest score climbs far beyond its first half tile's and the
    softmax reference is raised several times per row, in different half
    tiles for different rows of a wave (checked on the inputs first). Either
    one query tile over all keys (pieces=False, 700 keys) or a query tile
    whose 1,024 keys the schedule cuts into key-range pieces merged
    afterwards."""
    heads, rows = 2, 200
    H = heads * 128
    nk = 1024 if pieces else 700
    _say(f"attention online rescales pieces={pieces} keys={nk}")
    qb = I.normal_bf16("aresc.q", (rows, H), 8.0)
    k = O.bf16_to_f64(I.normal_bf16("aresc.k", (nk, H)))
    ramp = 1.0 + 3.0 * np.arange(nk) / nk
    ramp[-40:] *= 3.0
    kb = I.f32_to_bf16_bits((k * ramp[:, None]).astype(np.float32))
    vb = I.normal_bf16("aresc.v", (nk, H))
    cnt = _rescale_count(O.bf16_to_f64(qb), O.bf16_to_f64(kb))
    assert (cnt >= 2).mean() > 0.5 and cnt.max() >= 3, f"too few rescales: {np.bincount(cnt.ravel())}"
    assert _score_bound(O.bf16_to_f64(qb), O.bf16_to_f64(kb)) > 30.0
    q, k_d, v_d = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = poison((rows, H))
    if pieces:
        half = nk // 2
        h3.attention(q, q, q, o, rows, heads, groups=[(0, rows, [(k_d, v_d, 0, half), (k_d, v_d, half, nk - half)])])
    else:
        h3.attention(q, q, q, o, rows, heads, groups=[(0, rows, [(k_d, v_d, 0, nk)])])
    torch.cuda.synchronize()
    ref = O.attention_grouped(O.bf16_to_f64(qb), [(0, rows, [(O.bf16_to_f64(kb), O.bf16_to_f64(vb))])], heads, 128,
                              rows)
    assert_parity(f64(o), ref, "o")


def _score_bound(q_rows, k_rows):
    """The kernel's per-workgroup form choice, restated from its definition:
    |q| max|k| / sqrt(128) * log2(e) for the largest-norm query row. At most
    30 -> fixed softmax reference, above -> online form."""
    qn = np.sqrt(np.max(np.sum(q_rows.reshape(q_rows.shape[0], -1, 128) ** 2, axis=-1), axis=0))
    kn = np.sqrt(np.max(np.sum(k_rows.reshape(k_rows.shape[0], -1, 128) ** 2, axis=-1), axis=0))
    return float(np.max(qn * kn) / np.sqrt(128.0) * np.log2(np.e))


@pytest.mark.parametrize("q_scale,form", [(1.0, "fixed"), (5.0, "online")])
def test_attention_single_key_is_exact(q_scale, form):
    """One valid key: softmax weight exactly 1, so o equals that key's value
    bit for bit, on both softmax forms: q x 1
    keeps the score bound under 30 (fixed reference), q x 5 pushes it far
    above (online form)."""
    heads, L = 2, 64
    H = heads * 128
    qb, kb, vb = _qkv(L, heads, "a1", q_scale)
    B = _score_bound(O.bf16_to_f64(qb[:1]), O.bf16_to_f64(kb[:1]))
    assert (B <= 30.0) == (form == "fixed"), f"score bound {B:.1f} does not select the {form} form"
    o = poison((L, H))
    h3.attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, 1, heads)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o[:1]), vb[:1])
    assert_zero_rows(o, 1, "o")


@pytest.mark.parametrize("q_scale,form", [(1.0, "fixed"), (6.0, "online")])
def test_attention_many_queries_one_key_is_exact(q_scale, form):
    """Whole query tiles (300 rows, 42 heads: ragged second tile) attending to
    a single external key: every row's o equals that key's value bit for bit,
    on the fixed-reference and the online form."""
    heads, rows = 42, 300
    H = heads * 128
    qb = I.normal_bf16(f"a1m.q{q_scale}", (rows, H), q_scale)
    kb = I.normal_bf16("a1m.k", (1, H))
    vb = I.normal_bf16("a1m.v", (1, H))
    B = _score_bound(O.bf16_to_f64(qb), O.bf16_to_f64(kb))
    assert (B <= 30.0) == (form == "fixed"), f"score bound {B:.1f} does not select the {form} form"
    tk, tv = dev_bf16(kb), dev_bf16(vb)
    o = poison((rows, H))
    h3.attention(dev_bf16(qb), dev_bf16(np.zeros((rows, H), np.uint16)), dev_bf16(np.zeros((rows, H), np.uint16)),
                 o, rows, heads, groups=[(0, rows, [(tk, tv, 0, 1)])])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o), np.broadcast_to(vb, (rows, H)))


@pytest.mark.parametrize("segs,q_scale", [((320, 300), 1.0), ((130, 260, 70), 1.0), ((130, 260, 70), 8.0),
                                          ((64, 64, 64, 300), 1.0), ((500, 524), 1.0), ((500, 524), 8.0)])
def test_attention_key_range_pieces(segs, q_scale):
    """One query tile whose keys are several segments: the work schedule cuts
    it into key-range pieces (a piece may start exactly at a segment boundary
    or inside a segment, and end on a segment's ragged last tile), merged by
    the merge pass; also with peaked scores (q x 8: the online form, pieces
    with different row maxima)."""
    heads, rows = 1, 200
    H = heads * 128
    tiles = sum((n + 63) // 64 for n in segs)
    _say(f"attention pieces segs={segs} key tiles={tiles} q_scale={q_scale}")
    Lk = sum(segs)
    qb = I.normal_bf16("apc.q", (rows, H), q_scale)
    kb = I.normal_bf16("apc.k", (Lk, H))
    vb = I.normal_bf16("apc.v", (Lk, H))
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    # external segments of one K/V buffer, consecutive
    seg_list, begin = [], 0
    for n in segs:
        seg_list.append((k, v, begin, n))
        begin += n
    o = poison((rows, H))
    h3.attention(q, q, q, o, rows, heads, groups=[(0, rows, seg_list)])
    torch.cuda.synchronize()
    K, Vv = O.bf16_to_f64(kb), O.bf16_to_f64(vb)
    ref = O.attention_grouped(O.bf16_to_f64(qb), [(0, rows, [(K, Vv)])], heads, 128, rows)
    assert_parity(f64(o), ref, "o")


def test_attention_grouped_with_history():
    """Query groups over [external history ; own keys] segments; rows outside
    every group are zero (the streaming chunk's structure, scaled down)."""
    heads, L, V, Lh = 2, 600, 590, 300
    H = heads * 128
    qb, kb, vb = _qkv(L, heads, "ag")
    hk = I.normal_bf16("ag.hk", (Lh, H))
    hv = I.normal_bf16("ag.hv", (Lh, H))
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    tk, tv = dev_bf16(hk), dev_bf16(hv)
    groups = [(0, 64, [("self", 0, 200)]),
              (64, 100, [("self", 0, V)]),
              (150, 560, [(tk, tv, 20, 280), ("self", 0, V)]),
              (570, 590, [(tk, tv, 0, 1), ("self", 10, 50), ("self", 300, 3), (tk, tv, 299, 1)])]
    o = poison((L, H))
    h3.attention(q, k, v, o, V, heads, groups=groups)
    torch.cuda.synchronize()
    Q, K, Vv = O.bf16_to_f64(qb), O.bf16_to_f64(kb), O.bf16_to_f64(vb)
    HK, HV = O.bf16_to_f64(hk), O.bf16_to_f64(hv)
    og = [(0, 64, [(K[:200], Vv[:200])]),
          (64, 100, [(K[:V], Vv[:V])]),
          (150, 560, [(HK[20:300], HV[20:300]), (K[:V], Vv[:V])]),
          (570, 590, [(HK[0:1], HV[0:1]), (K[10:60], Vv[10:60]), (K[300:303], Vv[300:303]),
                      (HK[299:300], HV[299:300])])]
    ref = O.attention_grouped(Q[:V], og, heads, 128, V)
    got = f64(o)
    for (a, b, _) in og:
        assert_parity(got[a:b], ref[a:b], f"o[{a}:{b}]")
    for (a, b) in ((100, 150), (560, 570)):
        assert np.all(bits(o[a:b]) == 0), f"rows {a}:{b} outside every group must be zero"
    assert_zero_rows(o, V, "o")
    # the same history segments staged once by h3_kv_stage and read in place:
    # the same V^T planes and key norm maxima, so the same bits
    st = {(b, n): h3.kv_stage(tk[b:b + n], tv[b:b + n], heads) for (b, n) in ((20, 280), (0, 1), (299, 1))}
    groups_st = [(a, e, [(x[0], x[1], x[2], x[3], st[(x[2], x[3])]) if not isinstance(x[0], str) else x
                          for x in segs]) for (a, e, segs) in groups]
    o2 = poison((L, H))
    h3.attention(q, k, v, o2, V, heads, groups=groups_st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o2), bits(o))


@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_kv_stage_matches_attention_staging(q_scale):
    """h3_kv_stage's V^T plane and key norms equal what attention stages
    itself: a group reading only a staged external segment (longer than a
    K/V tile, ragged) gives the same bits as the unstaged call, on the fixed
    and the online softmax form, and matches the oracle."""
    heads, L, Lh = 3, 300, 777
    H = heads * 128
    qb = I.normal_bf16("kst.q", (L, H), q_scale)
    hk = I.normal_bf16("kst.hk", (Lh, H))
    hv = I.normal_bf16("kst.hv", (Lh, H))
    q, tk, tv = dev_bf16(qb), dev_bf16(hk), dev_bf16(hv)
    dummy = torch.zeros((L, H), dtype=torch.bfloat16, device="cuda")
    vt, km = h3.kv_stage(tk[5:705], tv[5:705], heads)
    torch.cuda.synchronize()
    # the key norm maxima: the largest squared norm of the BF16 key rows, per head
    kk = O.bf16_to_f64(hk[5:705]).reshape(700, heads, 128)
    np.testing.assert_allclose(km.cpu().numpy(), (kk ** 2).sum(-1).max(0), rtol=1e-5)
    outs = []
    for seg in ((tk, tv, 5, 700), (tk, tv, 5, 700, (vt, km))):
        o = poison((L, H))
        h3.attention(q, dummy, dummy, o, L, heads, groups=[(0, L, [seg])])
        torch.cuda.synchronize()
        outs.append(bits(o))
    np.testing.assert_array_equal(outs[1], outs[0])
    ref = O.attention(O.bf16_to_f64(qb), O.bf16_to_f64(hk[5:705]), O.bf16_to_f64(hv[5:705]), heads, 128)
    assert_parity(I.bf16_bits_to_f32(outs[1]).astype(np.float64), ref, "o (staged history)")
