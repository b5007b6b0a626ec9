"""FP64 CPU oracle of the H3 DiT block (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never does."""
from . import h3_oracle  # noqa: F401
