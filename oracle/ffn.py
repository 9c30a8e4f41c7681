"""Oracle: SwiGLU experts, FP4 expert weights and the layer forward.

Test infrastructure only (see the package docstring).

The layer output has a plain definition, computed here directly in float64
from the exact input values:

  y[t] = sum_{j} w[t,j] * FFN_{idx[t,j]}(x[t]) + FFN_shared(x[t])
  FFN(u) = W_down ( SiLU(clamp_g(W_gate u)) * clamp_v(W_up u) )

* SwiGLU: "From One Giant FFN to 384 Tiny Experts", Ch.1 (value branch
  W_up, gate branch W_gate, SiLU(x) = x * sigmoid(x), down projection).
* Routed + shared sum: same page, Ch.4 (DeepSeekMoE formula); the
  "moe-forward" excerpt of "DeepSeek-V3.2-Exp - Routing weights" (loop over
  experts, weighted add, shared expert added to every token); "DeepSeek
  V4.1 - Add shared" (Delta_ffn = y_routed + y_shared).
* Clamp: Ch.11.4 -- the value (linear) component clamped to [-L, L], the
  gate component capped above at L (L = swiglu_limit), before the product.
* FP4 experts: Ch.11.6 -- E2M1 values with one power-of-two scale per 1x32
  sub-block (OCP MXFP4).  Reading: the 32-blocks run along the input (K)
  dimension of each [out, in] weight row, two codes per byte with the even
  element in the low nibble, scale byte e meaning 2^(e-127).

The oracle returns float64; rounding to the output dtype is left to the
caller (the pages cast the fp32 sum back to the input dtype).

Pins: tests/test_oracle_ffn.py (E=1/top-1 reduces to a dense SwiGLU by plain
matmul, identical experts make the routed part (sum w) * SwiGLU(x), the
dense routing-map form over all experts agrees, clamp at L = inf is the
identity and a clamp-firing case against the closed form, the 16 E2M1 codes
against the published value set in tests/golden/e2m1_codes.json).
"""

import numpy as np


def _e2m1_value(code):
    """Value of a 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:                         # subnormal: 0 or 0.5
        mag = 0.5 * man
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return sign * mag


E2M1_VALUES = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def fp4_decode(packed, scales):
    """Dequantise FP4 weights.

    packed: uint8 [N, K/2]  (element 2i in the low nibble, 2i+1 in the high)
    scales: uint8 [N, K/32] (E8M0: value 2^(e-127); 255 is NaN)
    returns float64 [N, K]
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, half = packed.shape
    K = half * 2
    codes = np.empty((N, K), dtype=np.int64)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    vals = E2M1_VALUES[codes]
    sc = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    return vals * np.repeat(sc, 32, axis=1)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def swiglu_expert(u, w_gate, w_up, w_down, swiglu_limit=0.0):
    """One SwiGLU expert on rows u [n, d]; weights [I,d], [I,d], [d,I].

    swiglu_limit <= 0 (or inf) means no clamp.
    """
    u = np.asarray(u, dtype=np.float64)
    zg = u @ np.asarray(w_gate, dtype=np.float64).T       # gate branch
    zv = u @ np.asarray(w_up, dtype=np.float64).T         # value branch
    if swiglu_limit and np.isfinite(swiglu_limit) and swiglu_limit > 0:
        zg = np.minimum(zg, swiglu_limit)
        zv = np.clip(zv, -swiglu_limit, swiglu_limit)
    h = _silu(zg) * zv
    return h @ np.asarray(w_down, dtype=np.float64).T


def layer_forward(x, weights, indices, expert, shared=None, swiglu_limit=0.0):
    """Routed + shared forward for the tokens x [T, d].

    expert(e) -> (w_gate [I,d], w_up [I,d], w_down [d,I]) as float64 arrays
    (fetched one expert at a time so large layers fit in host memory);
    shared is the same triple or None.  Mirrors the page's loop: experts in
    ascending id order, each adding w * FFN_e(x[rows]) into an accumulator.
    """
    x = np.asarray(x, dtype=np.float64)
    indices = np.asarray(indices)
    weights = np.asarray(weights, dtype=np.float64)
    T, d = x.shape
    y = np.zeros((T, d), dtype=np.float64)
    for e in np.unique(indices):
        rows, slots = np.nonzero(indices == e)
        wg, wu, wd = expert(int(e))
        out = swiglu_expert(x[rows], wg, wu, wd, swiglu_limit)
        for r in range(rows.shape[0]):
            y[rows[r]] += weights[rows[r], slots[r]] * out[r]
    if shared is not None:
        wg, wu, wd = shared
        y += swiglu_expert(x, wg, wu, wd, swiglu_limit)
    return y


def dense_map_forward(x, G, expert, shared=None, swiglu_limit=0.0):
    """The same layer written with the dense routing map G [T, E]
    ("DeepSeek-V3.2-Exp - Routing weights": G is non-zero only for the
    selected experts): y[t] = sum over ALL experts e of G[t,e] FFN_e(x[t])."""
    x = np.asarray(x, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    y = np.zeros_like(x)
    for e in range(G.shape[1]):
        wg, wu, wd = expert(e)
        y += G[:, e:e + 1] * swiglu_expert(x, wg, wu, wd, swiglu_limit)
    if shared is not None:
        wg, wu, wd = shared
        y += swiglu_expert(x, wg, wu, wd, swiglu_limit)
    return y
