"""Oracle: MXFP8 activations for the FP4 expert layer (the FP8-compute variant).

Test infrastructure only (see the package docstring).

"From One Giant FFN to 384 Tiny Experts", Ch.11.6: the V4 experts are FP4
(E2M1) in OCP MXFP4 1x32 sub-blocks and are computed in FP8 (E4M3); the
released policy is FP4 experts, FP8 elsewhere.  The pages leave the
activation side of an FP8 expert GEMM open.  Reading taken here (the
MI355X-native form of "FP8 computation" on native FP4 weights): the
activations entering each routed expert GEMM (the gathered x for gate|up,
the SwiGLU output H for down) are quantised to OCP MXFP8 -- E4M3 elements,
one E8M0 scale per 32 consecutive inputs -- and the FP4 weights are used as
stored.  The shared expert (bf16 weights) keeps bf16 activations.

OCP MX rule for a block v_0..v_31: shared exponent X = floor(log2(max|v|)) - 8
(8 = the largest E4M3 exponent), clamped to the E8M0 range [-127, 127]; each
element is v / 2^X rounded to the nearest E4M3 value (ties to even mantissa)
and saturated to +-448.  An all-zero block gets X = 0.  E4M3 (OCP): bias 7,
normals 1.m x 2^(e-7) for e = 1..15 except the NaN codes S.1111.111,
subnormals m/8 x 2^-6.

The pages' training-time form of "computed in FP8" re-dequantises the FP4
weights to E4M3 in 128 x 128 blocks and states that the round trip is
lossless while the sub-block scale ratios stay within a bound
(fp4_to_fp8_blocks).  With the block scale chosen as the largest nonzero
sub-block scale over 2^6, every E2M1 value of a sub-block whose scale is at
most 2^14 below that maximum is an exact E4M3 value; larger spreads round.

Pins: tests/test_oracle_mx.py (the full E4M3 value table and the encoder's
round-half-even and saturation against torch's float8_e4m3fn cast,
hand-worked blocks, the bound |decode(q(v)) - v| <= 2^-4 |v| above the
subnormal range, and the layer against a per-token composition that
quantises with torch's E4M3 cast; the FP4 -> FP8 block re-dequantisation by
the exact round trip against fp4_decode at spreads up to 2^14, the first
lossy spread 2^15, and hand-worked codes).
"""

import math

import numpy as np

from .ffn import E2M1_VALUES

E4M3_MAX = 448.0


def _e4m3_value(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


_POS = E4M3_VALUES[:0x7F]                      # codes 0x00..0x7E: 0 .. 448, ascending


def e4m3_encode(a):
    """Nearest E4M3 codes to the reals in array a (ties: even code, i.e. even
    mantissa), saturating at +-448."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, mag, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    neg = np.signbit(a)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def mxfp8_quantize(v):
    """v [rows, K] (K % 32 == 0) -> (codes uint8 [rows, K], scales uint8 [rows, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    blk = v.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    # floor(log2(amax)) exactly: amax = f * 2^e with f in [0.5, 1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, (e - 1) - 8, 0).astype(np.float64)
    X = np.clip(X, -127, 127)
    codes = e4m3_encode(blk / (2.0 ** X)[:, :, None]).reshape(rows, K)
    return codes, (X + 127).astype(np.uint8)


def mxfp8_decode(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.int64)
    vals = E4M3_VALUES[codes]
    return vals * np.repeat(2.0 ** (scales - 127), 32, axis=1)


def fp4_to_fp8_blocks(packed, scales, block=128):
    """The FP4 -> FP8 re-dequantisation of one [N, K] weight matrix: E2M1 codes
    (two per byte, low nibble first) with one E8M0 scale per 32 inputs become
    E4M3 codes with one E8M0 scale per `block` x `block` block.

    Block scale byte B = max(s_max - 6, 0), s_max the largest scale byte among
    the block's 32-input sub-blocks that hold a nonzero code (127 for a block
    of zeros): the largest E2M1 magnitude 6 times 2^(s_max - B) = 384 fits
    E4M3.  Element code = nearest E4M3 value to e2m1 * 2^(s - B).  A block is
    lossless when every element's code decodes to exactly its FP4 value.

    Returns (codes uint8 [N, K], block_scales uint8 [N/block, K/block],
    lossless bool [N/block, K/block])."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.int64)
    N, K = packed.shape[0], packed.shape[1] * 2
    nib = np.empty((N, K), dtype=np.uint8)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    e2m1 = E2M1_VALUES[nib]
    nonzero_sub = (nib & 0x7).reshape(N, K // 32, 32).any(axis=2)
    codes = np.zeros((N, K), dtype=np.uint8)
    bsc = np.zeros((N // block, K // block), dtype=np.uint8)
    lossless = np.zeros((N // block, K // block), dtype=bool)
    sb = block // 32
    for bi in range(N // block):
        for bj in range(K // block):
            r = slice(bi * block, (bi + 1) * block)
            sub = scales[r, bj * sb:(bj + 1) * sb]
            nz = nonzero_sub[r, bj * sb:(bj + 1) * sb]
            s_max = int(sub[nz].max()) if nz.any() else 127
            B = max(s_max - 6, 0)
            c = slice(bj * block, (bj + 1) * block)
            v = e2m1[r, c] * 2.0 ** (np.repeat(sub, 32, axis=1) - B)
            q = e4m3_encode(v)
            codes[r, c] = q
            bsc[bi, bj] = B
            lossless[bi, bj] = bool(np.all(E4M3_VALUES[q] == v))
    return codes, bsc, lossless


def fp8_blocks_decode(codes, block_scales, block=128):
    """Values of E4M3 codes [N, K] with one E8M0 scale per block x block block."""
    codes = np.asarray(codes, dtype=np.uint8)
    bs = np.asarray(block_scales, dtype=np.int64)
    scale = np.repeat(np.repeat(2.0 ** (bs - 127), block, axis=0), block, axis=1)
    return E4M3_VALUES[codes] * scale


def _swiglu(h_g, h_u, limit):
    if limit > 0:
        h_g = np.minimum(h_g, limit)
        h_u = np.clip(h_u, -limit, limit)
    return h_g / (1.0 + np.exp(-h_g)) * h_u


def layer_forward_mx(x, weights, indices, expert, shared=None, swiglu_limit=0.0):
    """The routed + shared layer with MXFP8 activations on the routed experts:
    y[t] = sum_j w[t,j] * W_down,e dq(SwiGLU(W_gate,e dq(x_t), W_up,e dq(x_t)))
           + shared(x_t),  dq = MXFP8 quantise then decode (per token row)."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    y = np.zeros((T, d), dtype=np.float64)
    xq = mxfp8_decode(*mxfp8_quantize(x))
    for e in np.unique(indices):
        rows, slots = np.nonzero(indices == e)
        wg, wu, wd = expert(int(e))
        h = _swiglu(xq[rows] @ wg.T, xq[rows] @ wu.T, swiglu_limit)
        hq = mxfp8_decode(*mxfp8_quantize(h))
        out = hq @ wd.T
        for i in range(rows.shape[0]):
            y[rows[i]] += weights[rows[i], slots[i]] * out[i]
    if shared is not None:
        wg, wu, wd = shared
        y += _swiglu(x @ wg.T, x @ wu.T, swiglu_limit) @ wd.T
    return y
