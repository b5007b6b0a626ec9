"""Degenerate sizes through the C ABI on the GPU.

* No valid row (valid_len = 0 inside a 64-row buffer): every row is padding,
  so every output row is written +0.0 and nothing is read from the inputs,
  which are NaN/Inf-filled here. Checked for the block, the stack, dense
  attention, the linear projection and SwiGLU, each output buffer pre-filled
  with NaN.
* Empty buffer (L_buf = 0, null data pointers): the calls return H3_OK and
  launch nothing."""
import numpy as np
import pytest
import torch

from video_diffusion_transformer_dit_amd import h3
from video_diffusion_transformer_dit_amd import inputs as I

from util import bits, dev_bf16, poison

pytestmark = pytest.mark.gpu

L = 64


def _say(msg):
    print(msg, flush=True)


def _nan_inf(shape):
    """BF16 buffer of NaN and +Inf bit patterns (must never be read)."""
    t = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    t.view(-1)[::2] = float("inf")
    return t


def _tiny():
    s = I.TINY
    dims = h3.make_dims(s.hidden, s.heads, s.ffn, rot_dim=s.rot_dim, rope_theta=s.theta, eps=s.eps)
    w = {k: dev_bf16(v) for k, v in I.block_weights(s, "edge0").items()}
    mod = torch.from_numpy(I.mod_table(s, 1, tag="edge0.mod")).cuda()
    return s, dims, w, mod


def _all_zero(t):
    return bool(np.all(bits(t) == 0))


def test_no_valid_rows_writes_zero_everywhere():
    s, dims, w, mod = _tiny()
    weights = h3.make_weights(w)
    ws = torch.empty(h3.workspace_bytes(dims, L), dtype=torch.uint8, device="cuda")

    _say("block, valid_len = 0")
    x = _nan_inf((L, s.hidden))
    y = poison((L, s.hidden))
    h3.block_forward(dims, weights, x, y, mod, 1, 0, ws)
    torch.cuda.synchronize()
    assert _all_zero(y), "block output rows are not all +0.0"

    _say("stack of 2 blocks in place, valid_len = 0")
    xs = _nan_inf((L, s.hidden))
    arr = h3.make_weight_stack([weights, weights])
    h3.stack_forward(dims, arr, xs, mod, 0, 1, 0, ws)
    torch.cuda.synchronize()
    assert _all_zero(xs), "stack output rows are not all +0.0"

    H = s.heads * 128
    q, k, v = (_nan_inf((L, H)) for _ in range(3))
    _say("dense attention, valid_len = 0")
    o = poison((L, H))
    h3.attention(q, k, v, o, 0, s.heads)
    torch.cuda.synchronize()
    assert _all_zero(o), "attention output rows are not all +0.0"

    _say("linear, M_valid = 0")
    a = _nan_inf((L, 256))
    wl = dev_bf16(I.normal_bf16("edge0.wl", (512, 256), 0.02))
    c = poison((L, 512))
    h3.linear(a, wl, c, 0)
    torch.cuda.synchronize()
    assert _all_zero(c), "linear output rows are not all +0.0"

    _say("swiglu, valid_len = 0")
    u = _nan_inf((L, 2 * s.ffn))
    g = poison((L, s.ffn))
    h3.swiglu(u, g, 0, s.ffn)
    torch.cuda.synchronize()
    assert _all_zero(g), "swiglu output rows are not all +0.0"


def test_empty_buffers_launch_nothing():
    s, dims, w, mod = _tiny()
    weights = h3.make_weights(w)
    H = s.heads * 128
    empty = lambda cols: torch.empty((0, cols), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    _say("empty block, stack, attention, linear, swiglu")
    h3.block_forward(dims, weights, empty(s.hidden), empty(s.hidden), mod, 1, 0, ws)
    h3.stack_forward(dims, h3.make_weight_stack([weights]), empty(s.hidden), mod, 0, 1, 0, ws)
    h3.attention(empty(H), empty(H), empty(H), empty(H), 0, s.heads, workspace=ws)
    h3.linear(empty(256), dev_bf16(I.normal_bf16("edge1.wl", (512, 256), 0.02)), empty(512), 0)
    h3.swiglu(empty(2 * s.ffn), empty(s.ffn), 0, s.ffn)
    torch.cuda.synchronize()
