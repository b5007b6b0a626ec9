"""Seeded synthetic inputs shared by the HIP path and the oracle.

This module holds none of the block's arithmetic: it draws seeded normal
samples, stores them in BF16 or FP32 bit patterns, and describes the packed
token layouts of the workloads. Both sides receive the same bytes.

Recipe: master seed 20260903; each tensor draws from its own SFC64 stream whose
SeedSequence entropy is (master seed, CRC32 of the tensor's name). Samples are
drawn as float32 normals and cast to BF16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

MASTER_SEED = 20260903


def rng_for(name: str, seed: int = MASTER_SEED) -> np.random.Generator:
    """Independent SFC64 stream for one named tensor."""
    ss = np.random.SeedSequence([seed, zlib.crc32(name.encode())])
    return np.random.Generator(np.random.SFC64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest, ties to even:
    add 0x7FFF plus the lowest kept bit, then drop the low 16 bits. Inputs are
    finite normals, so NaN handling is not needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    t = np.right_shift(u, np.uint32(16))
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(t, u, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    return t.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_f32(name: str, shape, std: float = 1.0, mean: float = 0.0,
               seed: int = MASTER_SEED) -> np.ndarray:
    g = rng_for(name, seed)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def normal_bf16(name: str, shape, std: float = 1.0, mean: float = 0.0,
                seed: int = MASTER_SEED) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(name, shape, std, mean, seed))


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Width of one block and the packed sequence it runs over."""
    name: str
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    L_buf: int
    valid_len: int
    segments: tuple = ()          # ((label, rows), ...) of the packed sequence
    rot_dim: int = 64
    theta: float = 10000.0
    eps: float = 1e-6


# Tiny block the oracle finishes in well under a second: 512 rows
# [text 64 | audio 64 | video 384], 500 valid (12-row padding suffix).
TINY = BlockShape("tiny-512", 256, 2, 128, 1024, 512, 500,
                  (("text", 64), ("audio", 64), ("video", 384)))
# Full width at 4,096 valid tokens, no padding.
FULL_4096 = BlockShape("full-4096", 5376, 42, 128, 21504, 4096, 4096,
                       (("video", 4096),))
# Full width at the pages' packed length: 58,758 valid in a 58,816 buffer.
FULL_58816 = BlockShape("full-58816", 5376, 42, 128, 21504, 58816, 58758,
                        (("text", 512), ("audio", 1024), ("video", 57280)))


def scaled(shape: BlockShape, L_buf: int, valid_len: int | None = None,
           name: str | None = None) -> BlockShape:
    v = L_buf if valid_len is None else valid_len
    return dataclasses.replace(shape, L_buf=L_buf, valid_len=v,
                               name=name or f"{shape.name}@{L_buf}",
                               segments=(("video", L_buf),))


def block_weights(shape: BlockShape, tag: str = "blk0", w_std: float = 0.02,
                  gain_std: float = 0.02, bias: bool = False,
                  seed: int = MASTER_SEED) -> dict:
    """BF16 weight bit patterns of one block, [out, in] row-major.

    QK-norm gains are 1 + N(0, gain_std): gains drawn like the other weights would
    scale q and k to almost zero."""
    H, F, d = shape.hidden, shape.ffn, shape.head_dim
    w = {
        "w_qkv": normal_bf16(f"{tag}.w_qkv", (3 * H, H), w_std, seed=seed),
        "w_o": normal_bf16(f"{tag}.w_o", (H, H), w_std, seed=seed),
        "w_up": normal_bf16(f"{tag}.w_up", (2 * F, H), w_std, seed=seed),
        "w_down": normal_bf16(f"{tag}.w_down", (H, F), w_std, seed=seed),
        "q_gain": normal_bf16(f"{tag}.q_gain", (d,), gain_std, 1.0, seed=seed),
        "k_gain": normal_bf16(f"{tag}.k_gain", (d,), gain_std, 1.0, seed=seed),
    }
    if bias:
        w["b_qkv"] = normal_bf16(f"{tag}.b_qkv", (3 * H,), w_std, seed=seed)
        w["b_o"] = normal_bf16(f"{tag}.b_o", (H,), w_std, seed=seed)
        w["b_up"] = normal_bf16(f"{tag}.b_up", (2 * F,), w_std, seed=seed)
        w["b_down"] = normal_bf16(f"{tag}.b_down", (H,), w_std, seed=seed)
    return w


def activations(shape: BlockShape, tag: str = "x", std: float = 1.0,
                seed: int = MASTER_SEED) -> np.ndarray:
    """x [L_buf, H] BF16 bits, every row filled (padding rows too)."""
    return normal_bf16(tag, (shape.L_buf, shape.hidden), std, seed=seed)


def mod_table(shape: BlockShape, groups: int = 1, tag: str = "mod", std: float = 0.1,
              seed: int = MASTER_SEED) -> np.ndarray:
    """FP32 AdaLN table [groups, 6, H]."""
    return normal_f32(tag, (groups, 6, shape.hidden), std, seed=seed)


# Streaming chunk: [condition 256 | audio 128 | video 5 latents x 1,008 patches],
# video queries also read a pre-concatenated history of 15,120 rows.
STREAM_COND, STREAM_AUDIO, STREAM_VIDEO, STREAM_HISTORY = 256, 128, 5040, 15120


def streaming_shape(hidden=5376, heads=42, ffn=21504, cond=STREAM_COND, audio=STREAM_AUDIO,
                    video=STREAM_VIDEO) -> BlockShape:
    L = cond + audio + video
    return BlockShape(f"stream-{L}", hidden, heads, 128, ffn, L, L,
                      (("cond", cond), ("audio", audio), ("video", video)))


def history_kv(rows: int, hidden: int, tag: str = "hist", seed: int = MASTER_SEED):
    """History K and V, BF16 bits [rows, hidden] each, ~N(0, 1)."""
    return (normal_bf16(f"{tag}.k", (rows, hidden), seed=seed),
            normal_bf16(f"{tag}.v", (rows, hidden), seed=seed))
