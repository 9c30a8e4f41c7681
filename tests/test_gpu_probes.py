"""GPU checks of the roofline probes (moe_probe_read, moe_probe_mfma): every
shape launches and completes, reports the flops its launch performs, and
leaves the scratch output untouched (the probes store only when their
accumulated value hits a fixed constant, which the inputs never reach)."""

import pytest
import torch

from mixture_experts_ffn_route_amd import binding as B

pytestmark = pytest.mark.gpu

# shape -> (flops of one MFMA instruction, independent chains per wave)
SHAPES = {0: (16 * 16 * 32 * 2, 8), 1: (32 * 32 * 16 * 2, 8),
          2: (16 * 16 * 128 * 2, 16), 3: (16 * 16 * 128 * 2, 16)}


@pytest.mark.parametrize("shape", sorted(SHAPES))
def test_mfma_probe_flops_and_no_store(shape, gpu):
    out = torch.full((2048,), -7, dtype=torch.int32, device=gpu)
    iters = 3
    flops = B.moe_probe_mfma(iters, out, shape)
    torch.cuda.synchronize()
    per_inst, chains = SHAPES[shape]
    assert flops == 2048 * 4 * iters * chains * per_inst
    assert bool((out == -7).all()), "probe stored to its scratch output"


def test_read_probe_no_store(gpu):
    buf = torch.ones(16 << 20, dtype=torch.uint8, device=gpu)
    out = torch.full((1024,), -7, dtype=torch.int32, device=gpu)
    B.moe_probe_read(buf, out)
    torch.cuda.synchronize()
    assert bool((out == -7).all()), "probe stored to its scratch output"
