"""h3_mfma_ceiling, the matrix-core ceiling probe the benchmark times: it
launches one workgroup per CU, reports the flops it issues (BF16 and MXFP8
forms), writes a finite sum per thread, and rejects a sink smaller than 256
floats per CU."""
import numpy as np
import pytest
import torch

from video_diffusion_transformer_dit_amd import h3

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,k", [(h3.H3_CEIL_BF16, 16), (h3.H3_CEIL_FP8, 64)])
def test_mfma_ceiling_flops_and_sink(dtype, k):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"mfma ceiling probe: dtype {dtype}, {cus} CUs, 64 rounds", flush=True)
    sink = torch.full((cus * 256,), float("nan"), dtype=torch.float32, device="cuda")
    fl = h3.mfma_ceiling(64, sink, dtype)
    torch.cuda.synchronize()
    assert fl == cus * 4 * 64 * 16 * 2 * 32 * 32 * k
    assert np.all(np.isfinite(sink.cpu().numpy()))


def test_mfma_ceiling_rejects_a_small_sink():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((cus * 256 - 1,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(h3.H3Error) as e:
        h3.mfma_ceiling(64, sink)
    assert e.value.status == h3.H3_ERR_SHAPE
    torch.cuda.synchronize()
    assert torch.all(sink == 7.0).item()
