"""Pins of the oracle's MXFP8 activation quantiser and the MX layer forward
(the FP8-compute reading of "From One Giant FFN to 384 Tiny Experts",
Ch.11.6).  torch's float8_e4m3fn type serves as the independent E4M3
reference."""

import numpy as np
import pytest
import torch

import oracle
from oracle.mx import e4m3_encode


def test_e4m3_table_matches_torch():
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = bits.to(torch.float64).numpy()
    ours = oracle.E4M3_VALUES
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~finite)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0


def test_encode_matches_torch_rounding():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(size=20000) * 1e-2,
                        # exact midpoints between neighbouring codes (ties to even)
                        (oracle.E4M3_VALUES[1:0x7E] + oracle.E4M3_VALUES[2:0x7F]) / 2])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(v), ref)


def test_hand_worked_blocks():
    one = np.zeros((1, 32)); one[0, 0] = 1.0
    c, s = oracle.mxfp8_quantize(one)
    # amax 1 -> X = floor(log2 1) - 8 = -8 (scale byte 119); 1 / 2^-8 = 256 = 1.0 x 2^8 -> 0x78
    assert (s[0, 0], c[0, 0]) == (119, 0x78)
    sat = np.full((1, 32), 0.5); sat[0, 0] = 1.9
    c, s = oracle.mxfp8_quantize(sat)
    # 1.9 x 2^8 = 486.4 > 448 saturates; 0.5 x 2^8 = 128 = 1.0 x 2^7 -> 0x70
    assert s[0, 0] == 119 and c[0, 0] == 0x7E and np.all(c[0, 1:] == 0x70)
    z = np.zeros((2, 64))
    c, s = oracle.mxfp8_quantize(z)
    assert np.all(s == 127) and np.all(c == 0)


def test_error_bound():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(50, 256)) * np.exp(rng.uniform(-20, 20, size=(50, 1)))
    c, s = oracle.mxfp8_quantize(v)
    dq = oracle.mxfp8_decode(c, s)
    scale = np.repeat(2.0 ** (s.astype(np.int64) - 127), 32, axis=1)
    # normals: half an ulp (2^-4 relative); subnormals: half the 2^-9 step; saturated: <= 64/512
    bound = np.maximum(np.abs(v) * 2.0 ** -4, scale * 2.0 ** -10)
    sat = np.abs(v) / scale > 448
    assert np.all(np.abs(dq - v)[~sat] <= bound[~sat])
    assert np.all(np.abs(dq - v)[sat] <= 64 * scale[sat])


def _torch_mx(v):
    """Independent MXFP8 round trip with torch's E4M3 cast."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float64))
    rows, K = t.shape
    blk = t.reshape(rows, K // 32, 32)
    amax = blk.abs().amax(dim=2, keepdim=True)
    X = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, 1.0))) - 8,
                    torch.zeros_like(amax))
    q = (blk / 2.0 ** X).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * 2.0 ** X).reshape(rows, K).numpy()


def test_layer_forward_mx_against_an_independent_composition():
    rng = np.random.default_rng(2)
    T, d, I, E, k = 9, 64, 32, 4, 2
    x = rng.normal(size=(T, d))
    W = [(rng.normal(size=(I, d)) / 8, rng.normal(size=(I, d)) / 8, rng.normal(size=(d, I)) / 6)
         for _ in range(E)]
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1, size=(T, k))
    y = oracle.layer_forward_mx(x, w, idx, lambda e: W[e], None, 10.0)
    xq = _torch_mx(x)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            wg, wu, wd = W[idx[t, j]]
            g = np.minimum(xq[t] @ wg.T, 10.0)
            u = np.clip(xq[t] @ wu.T, -10.0, 10.0)
            h = g / (1 + np.exp(-g)) * u
            ref[t] += w[t, j] * (_torch_mx(h[None])[0] @ wd.T)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
