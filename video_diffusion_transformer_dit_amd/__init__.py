"""MI355X-native forward pass of the MiniMax-H3 DiT block.

The compute path is the C-ABI library ``libh3block.so`` (hand-written HIP
kernels for gfx950) under ``csrc/``; ``h3`` is its thin Python binding.
``inputs`` holds the seeded synthetic input generators."""
__all__ = ["inputs", "h3"]
