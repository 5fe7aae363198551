"""The MFMA rate probe behind the benchmark's measured peak: every wave's
check value is exactly 4 * iters (each of its 4 * iters MFMAs adds
16 * (1/16) * 1 = 1 to every accumulator element), for several grid sizes and
two calls in a row on one output buffer."""
import pytest
import torch

import paged_sparse_attention_amd as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,iters", [(1, 1), (64, 100), (600, 37)])
def test_probe_check_values(blocks, iters):
    out = torch.full((blocks * 4,), -1.0, dtype=torch.float32, device="cuda")
    P.oomb_probe_mfma_peak(blocks, iters, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 4.0 * iters))
    P.oomb_probe_mfma_peak(blocks, iters + 1, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 4.0 * (iters + 1)))
