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


# ---- FP4 -> FP8 re-dequantisation in 128 x 128 blocks ----

def _fp4_matrix(rng, N, K, scales):
    packed = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    return packed, np.asarray(scales, dtype=np.uint8)


def test_fp8_blocks_round_trip_is_exact_within_the_bound():
    """Every sub-block scale within 2^14 of its block's largest: the E4M3
    codes times the block scale give back the FP4 values exactly."""
    rng = np.random.default_rng(3)
    N, K = 256, 384
    top = rng.integers(100, 150, size=(N // 128, K // 128))
    spread = rng.integers(0, 15, size=(N, K // 32))
    scales = np.repeat(np.repeat(top, 128, axis=0), 4, axis=1) - spread
    packed, scales = _fp4_matrix(rng, N, K, scales)
    codes, bsc, lossless = oracle.fp4_to_fp8_blocks(packed, scales)
    assert lossless.all()
    np.testing.assert_array_equal(oracle.fp8_blocks_decode(codes, bsc),
                                  oracle.fp4_decode(packed, scales))
    # decode against torch's E4M3 values, independently of the oracle's table
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    scale = np.repeat(np.repeat(2.0 ** (bsc.astype(np.int64) - 127), 128, 0), 128, 1)
    np.testing.assert_array_equal(t * scale, oracle.fp4_decode(packed, scales))


def test_fp8_blocks_first_lossy_spread():
    """A spread of 2^15 pushes 0.5 and 1.5 of the small sub-block below E4M3's
    2^-9 step: those round (half to even) and the block is flagged."""
    N, K = 128, 128
    scales = np.full((N, K // 32), 140, dtype=np.uint8)
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    packed[0, 0] = 0x06                      # element (0, 0) = 4 in sub-block (0, 0), scale 140
    scales[1, 0] = 140 - 15
    packed[1, 0] = 0x31                      # (1, 0) = 0.5, (1, 1) = 1.5 at scale 125
    codes, bsc, lossless = oracle.fp4_to_fp8_blocks(packed, scales)
    assert bsc[0, 0] == 134 and not lossless[0, 0]
    # 0.5 * 2^-9 = 2^-10: halfway between 0 and 2^-9 -> code 0 (even)
    # 1.5 * 2^-9 = 3 * 2^-10: halfway between 1 and 2 (x 2^-9) -> code 2 (even)
    assert codes[1, 0] == 0x00 and codes[1, 1] == 0x02
    scales[1, 0] = 140 - 14
    codes, bsc, lossless = oracle.fp4_to_fp8_blocks(packed, scales)
    assert lossless[0, 0] and codes[1, 0] == 0x01 and codes[1, 1] == 0x03


def test_fp8_blocks_hand_worked():
    N, K = 128, 256
    scales = np.full((N, K // 32), 127, dtype=np.uint8)
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    packed[5, 0] = 0xD7                      # (5,0) = 6, (5,1) = -3, sub-block scale 127
    scales[9, 2] = 120
    packed[9, 32] = 0x01                     # (9,64) = 0.5, sub-block scale 120
    scales[20, 1] = 250                      # a sub-block of zeros does not set the block scale
    codes, bsc, lossless = oracle.fp4_to_fp8_blocks(packed, scales)
    # block scale 127 - 6 = 121: 6 * 2^6 = 384 = 1.5 * 2^8 -> 0x7C; -3 * 2^6 = -192 -> 0xF4;
    # 0.5 * 2^-1 = 2^-2 -> 0x28.  The all-zero second block column takes s_max = 127 too
    # (its scale-250 sub-block holds only zeros).
    assert bsc[0, 0] == 121 and bsc[0, 1] == 121 and lossless.all()
    assert (codes[5, 0], codes[5, 1], codes[9, 64]) == (0x7C, 0xF4, 0x28)
    assert np.count_nonzero(codes) == 3


def test_fp8_weight_layer_equals_fp4_layer_when_lossless():
    rng = np.random.default_rng(4)
    T, d, I, E, k = 7, 128, 128, 3, 2
    mats = []
    for _ in range(E):
        trio = []
        for (n, kk) in ((I, d), (I, d), (d, I)):
            sc = 120 + rng.integers(0, 6, size=(n, kk // 32))
            p, s = _fp4_matrix(rng, n, kk, sc)
            trio.append((p, s))
        mats.append(trio)
    fp4 = lambda e: tuple(oracle.fp4_decode(p, s) for p, s in mats[e])
    def fp8(e):
        out = []
        for p, s in mats[e]:
            c, b, ok = oracle.fp4_to_fp8_blocks(p, s)
            assert ok.all()
            out.append(oracle.fp8_blocks_decode(c, b))
        return tuple(out)
    x = rng.normal(size=(T, d))
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1, size=(T, k))
    np.testing.assert_array_equal(oracle.layer_forward_mx(x, w, idx, fp8, None, 10.0),
                                  oracle.layer_forward_mx(x, w, idx, fp4, None, 10.0))
