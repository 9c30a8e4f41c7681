"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: routing indices, counts and permutation bit-exact except tokens whose
k-th / (k+1)-th keys (or kept / dropped group scores, or two selected keys)
lie within 1e-6 relative; routing weights to 1e-5 relative; layer outputs
max|y - y_ref| / max|y_ref| <= 2e-2 (bf16), 5e-2 (FP4), 1e-4 (fp32).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu

SMALL = list(C.SMALL_WORKLOADS)


def _layer(workload, device):
    layer = synth.make_layer(workload, device)
    ora_table = None
    if workload.cfg.route_mode == "hash":
        cfg = workload.cfg
        table, _, _, _ = B.moe_build_tid2eid(layer["p"], cfg.n_routed_experts,
                                             cfg.n_activated_experts)
        ora_table, _, _, _ = oracle.tid2eid_greedy(layer["p"], cfg.n_routed_experts,
                                                   cfg.n_activated_experts)
        assert np.array_equal(table, ora_table)
        layer["tid2eid"] = torch.from_numpy(table).to(device)
    return layer, ora_table


def _forward(workload, layer, device, as_run=False):
    """moe_forward of the workload's layer (as_run: on the weights the workload
    runs with, i.e. FP8 re-dequantised ones where it asks for them)."""
    cfg, T = workload.cfg, workload.T
    if as_run:
        cfg, layer = H.run_weights(workload, cfg, layer, B)
    ws = B.alloc_workspace(cfg, T, device)
    y = torch.empty_like(layer["x"])
    print(f"[forward] {workload.name} T={T} ({cfg.expert_dtype} experts)", flush=True)
    B.moe_forward(cfg, layer, layer["x"], layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    return y, ws


@pytest.mark.parametrize("name", SMALL)
def test_route_small(name, gpu):
    wl = C.SMALL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    layer, ora_table = _layer(wl, gpu)
    w = torch.empty((T, cfg.n_activated_experts), dtype=torch.float32, device=gpu)
    idx = torch.empty((T, cfg.n_activated_experts), dtype=torch.int32, device=gpu)
    print(f"[route] {name}", flush=True)
    B.moe_route(cfg, layer, layer["x"], layer["token_ids"], T, w, idx)
    torch.cuda.synchronize()
    ow, oidx, aux = H.oracle_route(cfg, layer, ora_table)
    H.check_routing(cfg, H.cpu_np(w), H.cpu_np(idx), ow, oidx, aux, label=name)


@pytest.mark.parametrize("E,k,T,seed", [(16, 2, 64, 0), (64, 4, 301, 1), (256, 8, 4096, 2),
                                        (384, 8, 1000, 3), (1, 1, 17, 4), (1024, 3, 700, 5),
                                        (7, 7, 5, 6)])
def test_permute_random(E, k, T, seed, gpu):
    rng = np.random.default_rng(seed)
    indices = rng.integers(0, E, size=(T, k)).astype(np.int32)
    cfg = C.MoEConfig(dim=64, n_routed_experts=E, n_activated_experts=k, moe_inter_dim=64,
                      route_mode="hash", vocab_size=1)
    dev = lambda a: torch.from_numpy(a).to(gpu)
    idx = dev(indices)
    counts = torch.empty(E, dtype=torch.int32, device=gpu)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=gpu)
    st = torch.empty(T * k, dtype=torch.int32, device=gpu)
    ss = torch.empty(T * k, dtype=torch.int32, device=gpu)
    inv = torch.empty(T * k, dtype=torch.int32, device=gpu)
    flags = torch.zeros(4, dtype=torch.int32, device=gpu)
    print(f"[permute] E={E} k={k} T={T}", flush=True)
    B.moe_permute(cfg, idx, T, counts, offsets, st, ss, inv, flags)
    torch.cuda.synchronize()
    oc, oo, ost, oss, oinv = oracle.permute(indices, E)
    np.testing.assert_array_equal(H.cpu_np(counts), oc)
    np.testing.assert_array_equal(H.cpu_np(offsets), oo)
    np.testing.assert_array_equal(H.cpu_np(st), ost)
    np.testing.assert_array_equal(H.cpu_np(ss), oss)
    np.testing.assert_array_equal(H.cpu_np(inv).reshape(T, k), oinv)
    assert int(flags[0]) == 0


def test_permute_drops_out_of_range_ids(gpu):
    E, k, T = 8, 2, 50
    rng = np.random.default_rng(7)
    indices = rng.integers(0, E, size=(T, k)).astype(np.int32)
    indices[3, 1] = -1
    indices[10, 0] = E
    cfg = C.MoEConfig(dim=64, n_routed_experts=E, n_activated_experts=k, moe_inter_dim=64,
                      route_mode="hash", vocab_size=1)
    counts = torch.empty(E, dtype=torch.int32, device=gpu)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=gpu)
    st = torch.empty(T * k, dtype=torch.int32, device=gpu)
    ss = torch.empty(T * k, dtype=torch.int32, device=gpu)
    inv = torch.empty(T * k, dtype=torch.int32, device=gpu)
    flags = torch.zeros(4, dtype=torch.int32, device=gpu)
    B.moe_permute(cfg, torch.from_numpy(indices).to(gpu), T, counts, offsets, st, ss, inv, flags)
    torch.cuda.synchronize()
    valid = (indices >= 0) & (indices < E)
    oc, oo, ost, oss, oinv = oracle.permute(np.where(valid, indices, E), E + 1)
    np.testing.assert_array_equal(H.cpu_np(counts), oc[:E])
    assert int(offsets[E]) == valid.sum()
    inv_np = H.cpu_np(inv).reshape(T, k)
    assert inv_np[3, 1] == -1 and inv_np[10, 0] == -1
    np.testing.assert_array_equal(inv_np[valid], oinv[valid])
    assert int(flags[0]) & B.MOE_FLAG_EXPERT_RANGE


@pytest.mark.parametrize("E,k,T", [(6, 2, 2600), (13, 3, 2000), (64, 4, 1500)])
def test_forward_chunked_permutation(E, k, T, gpu):
    """Batches of more than 16 chunks of 256 pairs take the many-workgroup
    permutation inside moe_forward (per-chunk histograms, one scan wave per
    expert, the tile list from the expert totals); expert counts that are
    not multiples of 4 or 8 exercise the ragged ends of the per-expert and
    per-XCD splits.  Permutation bit-exact, tile list covering every expert's
    rows once, layer output against the oracle."""
    base = C.SMALL_WORKLOADS["hash_small"]
    wl = replace(base, name=f"hash_chunked_e{E}", T=T,
                 cfg=replace(base.cfg, n_routed_experts=E, n_activated_experts=k))
    cfg = wl.cfg
    assert T * k > 16 * 256
    layer, ora_table = _layer(wl, gpu)
    y, ws = _forward(wl, layer, gpu)
    v = B.workspace_views(cfg, T, ws)
    ow, oidx, aux = H.oracle_route(cfg, layer, ora_table)
    rc = H.check_routing(cfg, H.cpu_np(v["route_weights"]), H.cpu_np(v["route_indices"]),
                         ow, oidx, aux, label=wl.name)
    counts, offsets = H.cpu_np(v["counts"]), H.cpu_np(v["offsets"])
    st, ss, inv = H.cpu_np(v["sorted_tok"]), H.cpu_np(v["sorted_slot"]), H.cpu_np(v["inverse"])
    H.check_permutation_exact(rc.idx, E, counts, offsets, st, ss, inv)
    n = int(v["tile_count"][0])
    covered = np.zeros(E + 1, dtype=np.int64)
    for grp, row0, rows, _ in H.cpu_np(v["tiles"])[:n]:
        assert rows > 0 and 0 <= grp <= E
        if grp < E:
            assert offsets[grp] <= row0 and row0 + rows <= offsets[grp + 1]
        covered[grp] += rows
    np.testing.assert_array_equal(covered[:E], counts)
    assert covered[E] == T
    yref = H.oracle_forward(cfg, H.f64(layer["x"]), rc.ref_w, rc.idx, layer)
    H.check_layer_output(cfg, H.f64(y), yref, label=wl.name)
    assert int(v["flags"][0]) == 0


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(name, gpu):
    wl = C.SMALL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    layer, ora_table = _layer(wl, gpu)
    y, ws = _forward(wl, layer, gpu, as_run=True)
    v = B.workspace_views(cfg, T, ws)
    ow, oidx, aux = H.oracle_route(cfg, layer, ora_table)
    rc = H.check_routing(cfg, H.cpu_np(v["route_weights"]), H.cpu_np(v["route_indices"]),
                         ow, oidx, aux, label=name)
    counts, offsets = H.cpu_np(v["counts"]), H.cpu_np(v["offsets"])
    st, ss, inv = H.cpu_np(v["sorted_tok"]), H.cpu_np(v["sorted_slot"]), H.cpu_np(v["inverse"])
    H.check_permutation_valid(rc.idx, cfg.n_routed_experts, counts, offsets, st, ss, inv)
    H.check_permutation_exact(rc.idx, cfg.n_routed_experts, counts, offsets, st, ss, inv)
    yref = H.oracle_forward(cfg, H.f64(layer["x"]), rc.ref_w, rc.idx, layer, fp8=wl.fp8_weights)
    H.check_layer_output(cfg, H.f64(y), yref, label=name)
    assert int(v["flags"][0]) == 0


@pytest.mark.parametrize("name", [n for n, w in C.SMALL_WORKLOADS.items()
                                  if w.cfg.act_quant == "mxfp8"])
def test_mxfp8_activation_codes(name, gpu):
    """The workspace keeps x quantised to MXFP8.  x is the synthetic input, so
    its E4M3 codes and E8M0 shared exponents must equal the oracle's bit for
    bit (both sides scale by a power of two and round to nearest even)."""
    wl = C.SMALL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    layer, _ = _layer(wl, gpu)
    _, ws = _forward(wl, layer, gpu)
    v = B.workspace_views(cfg, T, ws)
    codes, scales = oracle.mxfp8_quantize(H.f64(layer["x"]))
    np.testing.assert_array_equal(H.cpu_np(v["xq_scales"]), scales)
    np.testing.assert_array_equal(H.cpu_np(v["xq"]), codes)


def test_forward_deterministic(gpu):
    wl = C.SMALL_WORKLOADS["v3_small"]
    layer, _ = _layer(wl, gpu)
    y1, _ = _forward(wl, layer, gpu)
    y2, _ = _forward(wl, layer, gpu)
    assert torch.equal(y1, y2)


def test_forward_t0_and_t1(gpu):
    wl = C.SMALL_WORKLOADS["v3_small"]
    cfg = wl.cfg
    layer, _ = _layer(wl, gpu)
    ws = B.alloc_workspace(cfg, 1, gpu)
    y = torch.full((1, cfg.dim), 7.0, dtype=torch.bfloat16, device=gpu)
    B.moe_forward(cfg, layer, layer["x"][:0], None, 0, y, ws)      # no-op
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    B.moe_forward(cfg, layer, layer["x"][:1], None, 1, y, ws)
    torch.cuda.synchronize()
    ow, oidx, _ = H.oracle_route(cfg, layer, rows=[0])
    yref = oracle.layer_forward(H.f64(layer["x"][:1]), ow, oidx, H.expert_fetcher(layer, cfg),
                                H.shared_weights(layer, cfg), cfg.swiglu_limit)
    assert H.max_rel_err(H.f64(y), yref) <= H.TOL["bf16"]


def test_forward_hash_skewed_multi_tile(gpu):
    """Every token hits the same k experts: rows per expert = T spans several
    GEMM tiles; the other experts get no rows."""
    base = C.SMALL_WORKLOADS["hash_small"]
    wl = C.Workload("hash_all_same", base.cfg, T=777)
    cfg, T = wl.cfg, wl.T
    layer = synth.make_layer(wl, gpu)
    k = cfg.n_activated_experts
    table = np.tile(np.array([3, 0, 9, 15][:k], dtype=np.int32), (cfg.vocab_size, 1))
    layer["tid2eid"] = torch.from_numpy(table).to(gpu)
    y, ws = _forward(wl, layer, gpu)
    v = B.workspace_views(cfg, T, ws)
    assert int(v["tile_count"][0]) > 2 * k
    ow, oidx, _ = oracle.hash_gate(H.cpu_np(layer["token_ids"]), table, cfg.route_scale) + (None,)
    yref = oracle.layer_forward(H.f64(layer["x"]), ow, oidx, H.expert_fetcher(layer, cfg),
                                H.shared_weights(layer, cfg))
    assert H.max_rel_err(H.f64(y), yref) <= H.TOL["bf16"]


@pytest.mark.parametrize("tiled", [False, True])
def test_forward_learned_skewed_multi_tile(tiled, gpu):
    """Learned routing where a large selection bias on the k experts of group 0
    makes every token pick them: each holds T rows over several GEMM tiles
    (tall tiles and ragged last tiles of one expert), the other experts get
    none, and the gate values stay the unbiased, renormalised scores."""
    base = C.SMALL_WORKLOADS["v3_small"]
    wl = C.Workload("v3_all_same", base.cfg, T=611, seed=7)
    cfg, T = wl.cfg, wl.T
    layer = synth.make_layer(wl, gpu)
    k, per_group = cfg.n_activated_experts, cfg.n_routed_experts // cfg.n_expert_groups
    assert k <= per_group
    bias = torch.zeros(cfg.n_routed_experts, dtype=torch.float32)
    bias[:k] = 10.0
    layer["gate_bias"] = bias.to(gpu)
    run_cfg, run_layer = B.pack_layer(cfg, layer) if tiled else (cfg, layer)
    ws = B.alloc_workspace(run_cfg, T, gpu)
    y = torch.empty_like(layer["x"])
    print(f"[forward] {wl.name} T={T} tiled={tiled}", flush=True)
    B.moe_forward(run_cfg, run_layer, layer["x"], None, T, y, ws)
    torch.cuda.synchronize()
    v = B.workspace_views(run_cfg, T, ws)
    counts = H.cpu_np(v["counts"])
    assert np.array_equal(counts[:k], np.full(k, T)) and counts[k:].sum() == 0
    assert int(v["tile_count"][0]) > 2 * k
    ow, oidx, aux = H.oracle_route(cfg, layer)
    rc = H.check_routing(cfg, H.cpu_np(v["route_weights"]), H.cpu_np(v["route_indices"]),
                         ow, oidx, aux, label=wl.name)
    yref = H.oracle_forward(cfg, H.f64(layer["x"]), rc.ref_w, rc.idx, layer)
    H.check_layer_output(cfg, H.f64(y), yref, label=wl.name)
    assert int(v["flags"][0]) == 0


def test_forward_hash_bad_token_id_flagged(gpu):
    wl = C.SMALL_WORKLOADS["hash_small"]
    cfg, T = wl.cfg, wl.T
    layer, _ = _layer(wl, gpu)
    layer["token_ids"] = layer["token_ids"].clone()
    layer["token_ids"][5] = cfg.vocab_size + 3
    y, ws = _forward(wl, layer, gpu)
    v = B.workspace_views(cfg, T, ws)
    assert int(v["flags"][0]) & B.MOE_FLAG_TOKEN_ID_RANGE
    assert torch.all(v["route_weights"][5] == 0)


def _mx_edge_rows(T, d, seed=11):
    """bf16-exact rows whose 32-input blocks put the MXFP8 quantiser on its
    edges: exact midpoints between neighbouring E4M3 codes (ties to even),
    values between 448 and 512 after scaling (saturation), subnormal
    midpoints, signed zeros, all-zero blocks and shared exponents at the
    [-127, 127] clamp (amax 2^-126 and 2^100)."""
    rng = np.random.default_rng(seed)
    vals = oracle.E4M3_VALUES[:0x7F].copy()                  # finite non-negative codes
    mids = (vals[:-1] + vals[1:]) / 2                        # includes subnormal midpoints
    big = vals[vals >= 4.0]
    sign = lambda n: rng.choice([-1.0, 1.0], size=n)
    to_bf16 = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    x = np.zeros((T, d), dtype=np.float64)
    for t in range(T):
        for b in range(d // 32):
            kind = (t * (d // 32) + b) % 5
            if kind == 4:
                continue                                     # all-zero block
            blk = rng.choice(mids, size=32) * sign(32)
            if kind == 1:
                blk = rng.choice(vals, size=32) * sign(32)
            if kind == 2:
                blk[1:8] = to_bf16(rng.uniform(448, 512, size=7)) * sign(7)
            if kind == 3:
                blk[2:6] = [0.0, -0.0, 0.0, -0.0]
            e = int(rng.integers(-20, 20))
            if (t + b) % 17 == 0:
                # amax 2^-120: the shared exponent -128 clamps to -127; every element
                # stays an fp32 normal
                e = -128
                blk = rng.choice(big, size=32) * sign(32)
            elif (t + b) % 17 == 1:
                e = 92                                       # amax near 2^100
            blk[0] = 256.0 + (rng.integers(0, 32) * 8)       # amax in [256, 512): X = e
            x[t, 32 * b:32 * b + 32] = np.ldexp(blk, e)
    return x


@pytest.mark.parametrize("name", ["fp4_mx_small"])
def test_mxfp8_codes_on_edge_values(name, gpu):
    """The quantiser's codes and shared exponents on crafted ties, saturation,
    subnormal and clamp cases, bit for bit against the oracle."""
    wl = C.SMALL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    layer, _ = _layer(wl, gpu)
    x64 = _mx_edge_rows(T, cfg.dim)
    xb = torch.from_numpy(x64).to(torch.bfloat16)
    assert np.array_equal(xb.double().numpy(), x64)            # exactly representable
    layer["x"] = xb.to(gpu)
    ws = B.alloc_workspace(cfg, T, gpu)
    y = torch.empty_like(layer["x"])
    print(f"[mx-edges] {name} T={T}", flush=True)
    B.moe_forward(cfg, layer, layer["x"], layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    v = B.workspace_views(cfg, T, ws)
    codes, scales = oracle.mxfp8_quantize(x64)
    np.testing.assert_array_equal(H.cpu_np(v["xq_scales"]), scales)
    np.testing.assert_array_equal(H.cpu_np(v["xq"]), codes)
    assert (scales == 0).any() and (scales == 127).any()       # clamp and all-zero blocks hit


_MX_NAMES = [n for n, w in C.SMALL_WORKLOADS.items() if w.cfg.act_quant == "mxfp8"]


@pytest.mark.parametrize("name,no_clamp", [(n, False) for n in _MX_NAMES] +
                         [("fp4_mx_clamp", True), ("fp8_mx_clamp", True)])
def test_mxfp8_hidden_codes(name, no_clamp, gpu):
    """The down GEMM's input: the routed rows of H in MXFP8, in permuted order.
    The gate|up GEMM writes them from its fp32 SwiGLU values at every tile
    height.  Against the oracle's float64 H of each
    permuted row (its expert's gate and up on the oracle-quantised x, through
    swiglu_expert with an identity down matrix):
    - every shared exponent equals the oracle's, or differs by one where the
      block maximum lies within 2^-7 relative of a power of two (the GEMM's
      rounding can put it on either side);
    - every decoded element equals the oracle's value, saturated at 448 times
      the GPU's block scale, to within half an E4M3 step (2^-4 relative, 2^(X-10)
      absolute below the normal range), and 1e-4 of the block maximum for the
      GEMM's fp32 sums.
    no_clamp: the same layer without the SwiGLU clamp (x ~ N(0, 20^2), so H
    reaches past the clamp's range), the layer output also checked against
    the oracle."""
    wl = C.SMALL_WORKLOADS[name]
    if no_clamp:
        wl = replace(wl, cfg=replace(wl.cfg, swiglu_limit=0.0))
    cfg, T = wl.cfg, wl.T
    k, I, E = cfg.n_activated_experts, cfg.moe_inter_dim, cfg.n_routed_experts
    layer, _ = _layer(wl, gpu)
    run_cfg, run_layer = H.run_weights(wl, cfg, layer, B)
    ws = B.alloc_workspace(run_cfg, T, gpu)
    y = torch.empty_like(layer["x"])
    tile_rows = B.moe_workspace_layout(run_cfg, T)["tile_rows"]
    print(f"[mx-hidden] {name} T={T} tile rows {tile_rows}", flush=True)
    B.moe_forward(run_cfg, run_layer, layer["x"], layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    v = B.workspace_views(run_cfg, T, ws)
    hq, hs = H.cpu_np(v["hq"]), H.cpu_np(v["hq_scales"])
    offsets, st = H.cpu_np(v["offsets"]), H.cpu_np(v["sorted_tok"])

    xd = oracle.mxfp8_decode(*oracle.mxfp8_quantize(H.f64(layer["x"])))
    get = H.expert_fetcher(layer, cfg, fp8=wl.fp8_weights)
    eye = np.eye(I)
    href = np.zeros((T * k, I))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            wg, wu, _ = get(e)
            href[r0:r1] = oracle.swiglu_expert(xd[st[r0:r1]], wg, wu, eye, cfg.swiglu_limit)

    _, osc = oracle.mxfp8_quantize(href)
    amax = np.abs(href).reshape(T * k, I // 32, 32).max(axis=2)
    with np.errstate(divide="ignore"):
        rel = np.abs(amax / np.exp2(np.round(np.log2(np.where(amax > 0, amax, 1.0)))) - 1.0)
    diff = hs.astype(np.int64) - osc.astype(np.int64)
    assert np.all(np.abs(diff) <= 1)
    assert np.all(rel[diff != 0] < 2.0 ** -7), "shared exponent off away from a power of two"
    assert (diff != 0).mean() < 0.01

    X = np.repeat(hs.astype(np.int64) - 127, 32, axis=1).astype(np.float64)
    lim = 448.0 * np.exp2(X)
    want = np.clip(href, -lim, lim)
    dec = oracle.mxfp8_decode(hq, hs)
    tol = (2.0 ** -4 * np.abs(want) + np.exp2(X - 10)
           + 1e-4 * np.repeat(amax, 32, axis=1))
    bad = np.abs(dec - want) > tol
    print(f"[mx-hidden] {name}: {int((diff != 0).sum())} exponents off by one, "
          f"{int(bad.sum())} elements out of bound", flush=True)
    assert not bad.any()
    if no_clamp:
        ow, oidx, aux = H.oracle_route(cfg, layer)
        rc = H.check_routing(cfg, H.cpu_np(v["route_weights"]), H.cpu_np(v["route_indices"]),
                             ow, oidx, aux, label=name)
        yref = H.oracle_forward(cfg, H.f64(layer["x"]), rc.ref_w, rc.idx, layer,
                                fp8=wl.fp8_weights)
        H.check_layer_output(cfg, H.f64(y), yref, label=f"{name} without the clamp")
