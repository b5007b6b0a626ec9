"""Helpers shared by the GPU tests: device transfer of BF16 bit patterns and the
parity metrics. No block arithmetic lives here."""
import numpy as np
import torch

from video_diffusion_transformer_dit_amd import inputs as I

# Parity bar: per output, relative Frobenius error <= 1e-2 and max |error| <= 5e-2
# of the reference's RMS (outputs are unit-variance-normalised by that RMS).
# Heavy-tailed intermediates (the SwiGLU product) are not unit-variance: there
# each element may additionally differ by BF16_SLACK * |reference|, i.e. four
# BF16 roundings (2^-9 each) of its own value, before the max bar applies.
REL_FRO = 1e-2
MAX_ABS = 5e-2
BF16_SLACK = 2.0 ** -7


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return I.bf16_bits_to_f32(bits(t)).astype(np.float64)


def poison(shape, dtype=torch.bfloat16) -> torch.Tensor:
    """Output buffer pre-filled with NaN, so unwritten elements are visible."""
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def metrics(got: np.ndarray, ref: np.ndarray, slack: float = 0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    if slack:
        err_max = np.maximum(np.abs(err) - slack * np.abs(ref), 0.0)
    else:
        err_max = np.abs(err)
    nref = np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mx = np.max(err_max) / rms if rms > 0 else np.max(err_max, initial=0.0)
    return float(rel), float(mx)


def assert_parity(got, ref, name, rel_tol=REL_FRO, max_tol=MAX_ABS, slack=0.0):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in GPU output"
    rel, mx = metrics(got, ref, slack)
    print(f"  parity {name}: rel_fro={rel:.3e} max_abs/rms={mx:.3e}", flush=True)
    assert rel <= rel_tol and mx <= max_tol, f"{name}: rel_fro={rel:.3e} max/rms={mx:.3e}"


def assert_zero_rows(t: torch.Tensor, r0: int, name: str):
    b = bits(t[r0:])
    assert np.all(b == 0), f"{name}: padding rows [{r0}, {t.shape[0]}) are not +0.0"
