"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random inputs; it holds none of the layer's
arithmetic.  Both the HIP path and the CPU oracle consume exactly the tensors
it returns (the oracle after copying them to the host), so the two sides see
the same bits.

Recipe (every tensor from its own generator, seeded by the workload seed and
the tensor's name, and per expert by its index):
  * x ~ N(0, x_scale^2), rounded to the activation dtype (round to nearest even);
  * gate weight ~ N(0, 1/dim); selection bias ~ U(-r, r) in fp32;
  * expert and shared weights ~ N(0, 1/fan_in) (fan_in = dim for W_gate and
    W_up, I for W_down);
  * FP4 routed experts: the fp32 draw is quantised to E2M1 with one E8M0
    scale per 32 inputs by the OCP MX rule (shared exponent
    floor(log2(amax)) - 2, nearest value with ties to even, saturating at 6);
  * hash routing: token frequencies p_i proportional to i^-s over the vocab
    (token id i-1 has rank i, so p is already sorted), T token ids sampled
    from p.
The generators run on the requested device (a CUDA device for the GPU
workloads, so multi-GB weights never touch the host).
"""

import zlib

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _seed(seed, *tags):
    words = [int(seed) & 0xFFFFFFFF]
    for t in tags:
        words.append(zlib.crc32(str(t).encode()) & 0xFFFFFFFF)
    state = np.random.SeedSequence(words).generate_state(2, dtype=np.uint32)
    return int(state[0]) | (int(state[1] & 0x7FFFFFFF) << 32)


def _gen(device, seed, *tags):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *tags))
    return g


def randn(shape, device, seed, *tags, std=1.0, dtype=torch.float32):
    g = _gen(device, seed, *tags)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def uniform(shape, device, seed, lo, hi, *tags):
    g = _gen(device, seed, *tags)
    v = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return v.mul_(hi - lo).add_(lo)


# E2M1 rounding boundaries between 0, .5, 1, 1.5, 2, 3, 4, 6 (midpoints)
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
# midpoints whose upper neighbour has the even (zero) mantissa bit
_E2M1_TIE_UP = (0.75, 1.75, 3.5)


def quantize_mxfp4(w):
    """fp32 [N, K] -> (packed uint8 [N, K/2], scales uint8 [N, K/32])."""
    N, K = w.shape
    assert K % 32 == 0
    blocks = w.reshape(N, K // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, exp = torch.frexp(amax)                       # amax = m * 2^exp, m in [0.5, 1)
    shared = (exp - 1 - 2).clamp(-127, 127)          # floor(log2 amax) - emax(e2m1)
    shared = torch.where(amax > 0, shared, torch.full_like(shared, -127))
    q = blocks / torch.ldexp(torch.ones_like(amax), shared.to(torch.float32)).unsqueeze(-1)
    mag = q.abs()
    mids = torch.tensor(_E2M1_MID, device=w.device, dtype=torch.float32)
    idx = torch.bucketize(mag, mids, right=False)
    for t in _E2M1_TIE_UP:
        idx = idx + (mag == t).to(idx.dtype)
    idx = idx.clamp(max=7)
    codes = idx + 8 * ((q < 0) & (idx > 0)).to(idx.dtype)
    codes = codes.reshape(N, K).to(torch.uint8)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    scales = (shared + 127).to(torch.uint8)
    return packed.contiguous(), scales.contiguous()


def zipf_probs(m, s):
    ranks = np.arange(1, m + 1, dtype=np.float64)
    p = ranks ** (-float(s))
    return p / p.sum()


def sample_token_ids(p, T, seed):
    rng = np.random.Generator(np.random.PCG64(_seed(seed, "token_ids")))
    return rng.choice(p.shape[0], size=T, p=p).astype(np.int32)


def make_layer(workload, device):
    """All inputs of a workload as tensors on `device` (dict).

    Keys: x, gate_w, gate_bias, w_gate, w_up, w_down, s_gate, s_up, s_down,
    sh_gate, sh_up, sh_down, token_ids, p (numpy float64, hash only).
    2-gram hash layers get token_ids [T, 2] = (previous id, current id): the
    batch is T / seq_len sequences of Zipf-sampled ids, and the first
    position of each sequence has previous id -1.
    Missing members are None.  workload.x_rows > T draws x with that many
    rows and keeps the first T (decode reuses the prefill batch's first rows).
    """
    cfg = workload.cfg
    seed = workload.seed
    T, d, E, I = workload.T, cfg.dim, cfg.n_routed_experts, cfg.moe_inter_dim
    adt = TORCH_DTYPE[cfg.act_dtype]
    out = dict.fromkeys(["x", "gate_w", "gate_bias", "w_gate", "w_up", "w_down", "s_gate",
                         "s_up", "s_down", "sh_gate", "sh_up", "sh_down", "token_ids", "p"])
    rows = max(T, workload.x_rows)
    out["x"] = randn((rows, d), device, seed, "x", d, std=workload.x_scale, dtype=adt)[:T].contiguous()
    if cfg.route_mode == "learned":
        out["gate_w"] = randn((E, d), device, seed, "gate_w", E, d, std=d ** -0.5, dtype=adt)
        if cfg.has_bias:
            r = workload.bias_range
            out["gate_bias"] = uniform((E,), device, seed, -r, r, "gate_bias", E)
    else:
        p = zipf_probs(cfg.vocab_size, workload.zipf_s)
        out["p"] = p
        ids = sample_token_ids(p, T, seed)
        if cfg.route_mode == "ngram":
            L = workload.seq_len or T
            prev = np.concatenate([[-1], ids[:-1]]).astype(np.int32)
            prev[::L] = -1
            ids = np.stack([prev, ids], axis=1)
        out["token_ids"] = torch.from_numpy(np.ascontiguousarray(ids)).to(device)

    shapes = {"w_gate": (I, d), "w_up": (I, d), "w_down": (d, I)}
    for name, (n_out, n_in) in shapes.items():
        std = n_in ** -0.5
        if cfg.expert_dtype == "fp4":
            packed = torch.empty((E, n_out, n_in // 2), dtype=torch.uint8, device=device)
            scales = torch.empty((E, n_out, n_in // 32), dtype=torch.uint8, device=device)
            for e in range(E):
                w = randn((n_out, n_in), device, seed, name, e, n_out, n_in, std=std)
                packed[e], scales[e] = quantize_mxfp4(w)
            out[name] = packed
            out["s_" + name[2:]] = scales
        else:
            t = torch.empty((E, n_out, n_in), dtype=TORCH_DTYPE[cfg.expert_dtype], device=device)
            for e in range(E):
                t[e] = randn((n_out, n_in), device, seed, name, e, n_out, n_in, std=std,
                             dtype=t.dtype)
            out[name] = t
        if cfg.n_shared_experts:
            out["sh_" + name[2:]] = randn((n_out, n_in), device, seed, "sh_" + name, n_out, n_in,
                                          std=std, dtype=adt)
    return out
