"""GPU tests of the FP4 -> FP8 re-dequantisation (moe_redequant_fp8) against
the oracle's, bit for bit: E4M3 codes (read back from the FP8 expert layout
with numpy reshapes), E8M0 block scales and lossy flags, on matrices whose
128 x 128 blocks span sub-block scale spreads below, at and past the lossless
bound, blocks of zeros, zero sub-blocks with stray scales, and block scales
that floor at 0."""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_route_amd import binding as B

pytestmark = pytest.mark.gpu


def _unpack(fp8, n_mat, N, K):
    """FP8 expert layout -> [n_mat, N, K]: block (nb, st) of 2 KB holds
    (h, q, c, i) -> row 16nb + c, input 128st + 64h + 16q + i."""
    p = fp8.reshape(n_mat, N // 16, K // 128, 2, 4, 16, 16)       # mat nb st h q c i
    return p.transpose(0, 1, 5, 2, 3, 4, 6).reshape(n_mat, N, K)


def _fp4_inputs(seed, n_mat, N, K):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n_mat, N, K // 2)).astype(np.uint8)
    top = rng.integers(100, 150, size=(n_mat, N // 128, K // 128))
    spread = rng.integers(0, 12, size=(n_mat, N, K // 32))
    wide = rng.random(size=spread.shape) < 0.002                 # a few spreads past 14
    spread = np.where(wide, rng.integers(14, 20, size=spread.shape), spread)
    scales = np.repeat(np.repeat(top, 128, axis=1), 4, axis=2) - spread
    zero_sub = rng.random(size=(n_mat, N, K // 32)) < 0.01       # zero sub-blocks, stray scales
    codes.reshape(n_mat, N, K // 32, 16)[zero_sub] = 0x80        # +0 and -0 nibbles
    scales[zero_sub] = 250
    codes[0, :128, :64] = 0                                      # one all-zero block
    scales[1, 128:, 4:8] = rng.integers(0, 5, size=(N - 128, 4)) # block scale floors at 0
    return codes, scales.astype(np.uint8)


@pytest.mark.parametrize("seed,n_mat,N,K", [(0, 3, 256, 384), (1, 2, 384, 256)])
def test_redequant_matches_oracle(seed, n_mat, N, K, gpu):
    codes, scales = _fp4_inputs(seed, n_mat, N, K)
    dev = lambda a: torch.from_numpy(a).to(gpu)
    fp8 = torch.empty((n_mat * N * K,), dtype=torch.uint8, device=gpu)
    bsc = torch.empty((n_mat, N // 128, K // 128), dtype=torch.uint8, device=gpu)
    lossy = torch.empty_like(bsc)
    print(f"[fp8] redequant seed={seed} {n_mat}x{N}x{K}", flush=True)
    B.moe_redequant_fp8(dev(codes), dev(scales), n_mat, N, K, fp8, bsc, lossy)
    torch.cuda.synchronize()
    got = _unpack(fp8.cpu().numpy(), n_mat, N, K)
    n_lossy = 0
    for m in range(n_mat):
        oc, ob, ol = oracle.fp4_to_fp8_blocks(codes[m], scales[m])
        np.testing.assert_array_equal(bsc[m].cpu().numpy(), ob)
        np.testing.assert_array_equal(lossy[m].cpu().numpy(), (~ol).astype(np.uint8))
        np.testing.assert_array_equal(got[m], oc)
        n_lossy += int((~ol).sum())
    assert 0 < n_lossy < bsc.numel()        # both kinds of block were exercised


def test_redequant_zero_matrices_is_a_no_op(gpu):
    fp8 = torch.full((16,), 7, dtype=torch.uint8, device=gpu)
    B.moe_redequant_fp8(None, None, 0, 128, 128, fp8, fp8, fp8)
    torch.cuda.synchronize()
    assert torch.all(fp8 == 7)
