"""The precision-preserving LoRA consumer variants (Sol-H3 report, §3.5
"Precision-preserving LoRA fusion"): the consumer forms bf16(base + delta)
itself, so the result must equal, bit for bit, storing that rounded sum and
running the plain consumer on it; and it must match the FP64 oracle. Inputs
include deltas of exactly half a BF16 spacing, so every rounding tie is hit.
All calls go through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import h3_oracle as O
from video_diffusion_transformer_dit_amd import h3
from video_diffusion_transformer_dit_amd import inputs as I

from util import BF16_SLACK, assert_parity, assert_zero_rows, bits, dev_bf16, dev_f32, dev_i32, f64, poison

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _delta_bits(name, base_bits, std=0.05, ties=False):
    """A LoRA delta: N(0, std) in BF16, or (ties) exactly half the BF16 spacing
    of the base element with a random sign, so base + delta is a tie."""
    if not ties:
        return I.normal_bf16(name, base_bits.shape, std)
    b = I.bf16_bits_to_f32(base_bits).astype(np.float64)
    e = np.frexp(np.where(b == 0, 1.0, b))[1]          # |b| in [2^(e-1), 2^e)
    half = np.ldexp(1.0, e - 9)                           # half of the spacing 2^(e-8)
    sign = np.where(I.rng_for(name).integers(0, 2, size=b.shape) == 0, -1.0, 1.0)
    return I.f32_to_bf16_bits((sign * half).astype(np.float32))


def _rounded_sum(base: torch.Tensor, delta: torch.Tensor) -> torch.Tensor:
    """The unfused sequence's stored sum: bf16(base + delta) (torch rounds to nearest even)."""
    return (base.float() + delta.float()).to(torch.bfloat16)


@pytest.mark.parametrize("F,L,V", [(1024, 300, 291), (21504, 20, 19), (8, 3, 3)])
@pytest.mark.parametrize("ties", [False, True])
def test_swiglu_lora(F, L, V, ties):
    _say(f"swiglu_lora F={F} L={L} V={V} ties={ties}")
    ub = I.normal_bf16("swl.u", (L, 2 * F), 2.0)
    db = _delta_bits("swl.d", ub, ties=ties)
    u, du = dev_bf16(ub), dev_bf16(db)
    g = poison((L, F))
    h3.swiglu_lora(u, du, g, V, F)
    g_ref = poison((L, F))
    h3.swiglu(_rounded_sum(u, du), g_ref, V, F)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(g), bits(g_ref))
    s = O.lora_input(O.bf16_to_f64(ub[:V]), O.bf16_to_f64(db[:V]))
    assert_parity(f64(g)[:V], O.swiglu(s, F), "g", slack=BF16_SLACK)
    assert_zero_rows(g, V, "g")


@pytest.mark.parametrize("heads,L,V", [(2, 300, 291), (42, 40, 37)])
@pytest.mark.parametrize("with_v", [False, True])
@pytest.mark.parametrize("ties", [False, True])
def test_qk_norm_rope_lora(heads, L, V, with_v, ties):
    _say(f"qk_norm_rope_lora heads={heads} L={L} V={V} v={with_v} ties={ties}")
    H = heads * 128
    qkv_b = I.normal_bf16("qkl.qkv", (L, 3 * H), 3.0)
    d_b = _delta_bits("qkl.d", qkv_b, std=0.3, ties=ties)
    gq = dev_bf16(I.normal_bf16("qkl.gq", (128,), 0.02, 1.0))
    gk = dev_bf16(I.normal_bf16("qkl.gk", (128,), 0.02, 1.0))
    posv = I.rng_for("qkl.pos").integers(0, 60000, size=L).astype(np.int32)
    pos = dev_i32(posv)
    qkv, d = dev_bf16(qkv_b), dev_bf16(d_b)
    h3.qk_norm_rope_lora(qkv[:, :H], qkv[:, H:2 * H], d[:, :H], d[:, H:2 * H], gq, gk, V, heads,
                         v=qkv[:, 2 * H:] if with_v else None, dv=d[:, 2 * H:] if with_v else None, pos=pos)
    ref = _rounded_sum(dev_bf16(qkv_b), d)
    h3.qk_norm_rope(ref[:, :H], ref[:, H:2 * H], gq, gk, V, heads, pos=pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(qkv[:, :2 * H]), bits(ref[:, :2 * H]))
    if with_v:
        np.testing.assert_array_equal(bits(qkv[:V, 2 * H:]), bits(ref[:V, 2 * H:]))
        assert_zero_rows(qkv[:, 2 * H:], V, "v")
    else:
        np.testing.assert_array_equal(bits(qkv[:, 2 * H:]), qkv_b[:, 2 * H:])
    s = O.lora_input(O.bf16_to_f64(qkv_b[:V]), O.bf16_to_f64(d_b[:V]))
    got = f64(qkv)
    for name, sl, g in (("q", slice(0, H), gq), ("k", slice(H, 2 * H), gk)):
        r = O.qk_norm_rope(s[:, sl], posv[:V], heads, 128, f64(g), 1e-6, 64, 1e4, 0)
        assert_parity(got[:V, sl], r, name)
        assert_zero_rows(qkv[:, sl], V, name)


@pytest.mark.parametrize("H,L,V", [(256, 300, 291), (5376, 70, 67)])
@pytest.mark.parametrize("gate_bf16", [False, True])
@pytest.mark.parametrize("with_h", [True, False])
@pytest.mark.parametrize("ties", [False, True])
def test_modnorm_lora(H, L, V, gate_bf16, with_h, ties):
    _say(f"modnorm_lora H={H} L={L} V={V} gate_bf16={gate_bf16} h={with_h} ties={ties}")
    G = 3
    xb = I.normal_bf16("mnl.x", (L, H))
    bb = I.normal_bf16("mnl.b", (L, H))
    db = _delta_bits("mnl.d", bb, ties=ties)
    mod = I.normal_f32("mnl.mod", (G, 6, H), 0.3)
    idx = I.rng_for("mnl.idx").integers(0, G, size=L).astype(np.int32)
    x, br, d, md, ix = dev_bf16(xb), dev_bf16(bb), dev_bf16(db), dev_f32(mod), dev_i32(idx)
    x1 = poison((L, H))
    h = poison((L, H)) if with_h else None
    h3.fused_modulate_norm_lora(x, br, d, md[:, 2], x1, V, shift=md[:, 0] if with_h else None,
                                scale=md[:, 1] if with_h else None, h_out=h, gate_bf16=gate_bf16,
                                ld_mod_group=6 * H, n_mod_groups=G, mod_idx=ix)
    # the unfused sequence
    s = _rounded_sum(br, d)
    x1_ref, h_ref = poison((L, H)), poison((L, H))
    if not gate_bf16:
        h3.fused_modulate_norm(x, md[:, 0], md[:, 1], h_ref, V, branch=s, gate=md[:, 2], x1_out=x1_ref,
                               ld_mod_group=6 * H, n_mod_groups=G, mod_idx=ix)
    else:
        gate_rows = md[:, 2][ix.long()]                                    # [L, H] FP32
        p = (gate_rows * s.float()).to(torch.bfloat16)                     # the BF16 gate product
        x1_ref = (x.float() + p.float()).to(torch.bfloat16)
        x1_ref[V:] = 0
        h3.fused_modulate_norm(x1_ref, md[:, 0], md[:, 1], h_ref, V, ld_mod_group=6 * H, n_mod_groups=G,
                               mod_idx=ix)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(x1), bits(x1_ref))
    if with_h:
        np.testing.assert_array_equal(bits(h), bits(h_ref))
    # the oracle
    m = O.gather_mod(mod.astype(np.float64), idx, V)
    sv = O.lora_input(O.bf16_to_f64(bb[:V]), O.bf16_to_f64(db[:V]))
    xv = O.bf16_to_f64(xb[:V])
    z = (O.gated_residual_bf16_product(xv, m[:, O.GATE_A], sv) if gate_bf16
         else O.gated_residual(xv, m[:, O.GATE_A], sv))
    assert_parity(f64(x1)[:V], z, "x1")
    assert_zero_rows(x1, V, "x1")
    if with_h:
        assert_parity(f64(h)[:V], O.modulate_norm(z, m[:, O.SHIFT_A], m[:, O.SCALE_A], 1e-6, 0), "h")
        assert_zero_rows(h, V, "h")


def test_lora_consumers_full_size_bit_exact():
    """At the block's full sizes (58,816 buffer rows, 58,758 valid): the three
    fused consumers equal the unfused sequence bit for bit (compared on the GPU)."""
    _say("lora consumers full size")
    L, V, H, heads, F = 58816, 58758, 5376, 42, 21504
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260903)

    def rnd(shape, std=1.0):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    def same(a, b, name):
        eq = torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
        assert eq, f"{name}: fused and unfused differ"

    # QKV consumer
    qkv, dq = rnd((L, 3 * H), 3.0), rnd((L, 3 * H), 0.3)
    gq, gk = (1 + rnd((128,), 0.02).float()).to(torch.bfloat16), (1 + rnd((128,), 0.02).float()).to(torch.bfloat16)
    ref = _rounded_sum(qkv, dq)
    h3.qk_norm_rope(ref[:, :H], ref[:, H:2 * H], gq, gk, V, heads)
    h3.qk_norm_rope_lora(qkv[:, :H], qkv[:, H:2 * H], dq[:, :H], dq[:, H:2 * H], gq, gk, V, heads,
                         v=qkv[:, 2 * H:], dv=dq[:, 2 * H:])
    torch.cuda.synchronize()
    same(qkv[:, :2 * H], ref[:, :2 * H], "qk")
    same(qkv[:V, 2 * H:], ref[:V, 2 * H:], "v")
    del qkv, dq, ref
    # residual-modulation consumer
    x, br, d = rnd((L, H)), rnd((L, H)), rnd((L, H), 0.05)
    mod = torch.randn((1, 6, H), generator=gen, device="cuda") * 0.3
    x1, h, x1r, hr = (torch.empty((L, H), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    h3.fused_modulate_norm_lora(x, br, d, mod[:, 2], x1, V, shift=mod[:, 0], scale=mod[:, 1], h_out=h,
                                ld_mod_group=6 * H)
    h3.fused_modulate_norm(x, mod[:, 0], mod[:, 1], hr, V, branch=_rounded_sum(br, d), gate=mod[:, 2], x1_out=x1r,
                           ld_mod_group=6 * H)
    torch.cuda.synchronize()
    same(x1, x1r, "x1")
    same(h, hr, "h")
    del x, br, d, x1, h, x1r, hr
    # SwiGLU consumer
    u, du = rnd((L, 2 * F), 2.0), rnd((L, 2 * F), 0.05)
    g, gr = (torch.empty((L, F), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    h3.swiglu_lora(u, du, g, V, F)
    h3.swiglu(_rounded_sum(u, du), gr, V, F)
    torch.cuda.synchronize()
    same(g, gr, "g")
