"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same entry point, same token count, hence the same tile
and kernel choices).

bf16 and FP4 layers run on tiled weights (moe_pack_weights), as the
benchmark does, and must match the row layout bit for bit.
Routing and the permutation are compared for every token.  The layer output
is compared on a sample of tokens the float64 oracle computes one by one
(first, last and seeded random positions; every token for the decode batch
and the tiny fp32 layer).  Bars as in the small parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu

# tokens whose output the oracle recomputes (None: all of them)
SAMPLE = {"tiny_fp32": None, "v3_decode": None, "hash_bf16": 64, "v3_prefill": 24,
          "v41_flash_fp4": 16, "ngram_bf16": 64, "v41_flash_fp4_mx": 16, "v41_flash_fp8": 16}


def _sample_rows(T, n, seed):
    if n is None or n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], mid]))


@pytest.mark.parametrize("name", list(C.FULL_WORKLOADS))
def test_forward_full_size(name, gpu):
    wl = C.FULL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    print(f"[full] {name}: generating T={T} d={cfg.dim} E={cfg.n_routed_experts}", flush=True)
    layer = synth.make_layer(wl, gpu)
    ora_table = None
    if cfg.route_mode == "hash":
        table, _, _, _ = B.moe_build_tid2eid(layer["p"], cfg.n_routed_experts,
                                             cfg.n_activated_experts)
        ora_table, _, _, _ = oracle.tid2eid_greedy(layer["p"], cfg.n_routed_experts,
                                                   cfg.n_activated_experts)
        np.testing.assert_array_equal(table, ora_table)
        layer["tid2eid"] = torch.from_numpy(table).to(gpu)
    ws = B.alloc_workspace(cfg, T, gpu)
    y = torch.empty_like(layer["x"])
    if wl.fp8_weights:
        print(f"[full] {name}: re-dequantising the FP4 experts to FP8", flush=True)
        run_cfg, run_layer = H.run_weights(wl, cfg, layer, B)
    elif cfg.act_dtype == "bf16":
        print(f"[full] {name}: packing the expert weights", flush=True)
        run_cfg, run_layer = B.pack_layer(cfg, layer)
    else:
        run_cfg, run_layer = cfg, layer
    print(f"[full] {name}: forward ({run_cfg.weight_layout} weights)", flush=True)
    B.moe_forward(run_cfg, run_layer, layer["x"], layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    v = B.workspace_views(cfg, T, ws)
    assert int(v["flags"][0]) == 0
    if run_cfg is not cfg and not wl.fp8_weights:
        y_rows = torch.empty_like(y)
        ws_rows = B.alloc_workspace(cfg, T, gpu)
        B.moe_forward(cfg, layer, layer["x"], layer["token_ids"], T, y_rows, ws_rows)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_rows.view(torch.int16))
        del y_rows, ws_rows, run_layer

    if wl.fp8_weights:
        del run_layer
    # routing of every token
    print(f"[full] {name}: oracle routing", flush=True)
    ow, oidx, aux = H.oracle_route(cfg, layer, ora_table)
    gidx = H.cpu_np(v["route_indices"])
    differ = H.compare_routing(cfg, H.cpu_np(v["route_weights"]), gidx, ow, oidx, aux)

    # permutation of every row: properties, and equality with the oracle's
    # permutation of its own routing when the routings agree
    counts, offsets = H.cpu_np(v["counts"]), H.cpu_np(v["offsets"])
    st, ss, inv = H.cpu_np(v["sorted_tok"]), H.cpu_np(v["sorted_slot"]), H.cpu_np(v["inverse"])
    H.check_permutation_valid(gidx, cfg.n_routed_experts, counts, offsets, st, ss, inv)
    if not differ.any():
        oc, oo, ost, oss, oinv = oracle.permute(oidx, cfg.n_routed_experts)
        np.testing.assert_array_equal(counts, oc)
        np.testing.assert_array_equal(offsets, oo)
        k = cfg.n_activated_experts
        np.testing.assert_array_equal(st[:T * k], ost)
        np.testing.assert_array_equal(ss[:T * k], oss)
        np.testing.assert_array_equal(inv.reshape(T, k), oinv)

    # layer output on the sampled tokens
    rows = _sample_rows(T, SAMPLE[name], seed=T)
    rows = rows[~differ[rows]]
    print(f"[full] {name}: oracle forward of {rows.size} tokens", flush=True)
    x_rows = H.f64(layer["x"][torch.as_tensor(rows, device=gpu)])
    yref = H.oracle_forward(cfg, x_rows, ow[rows], oidx[rows], layer, fp8=wl.fp8_weights)
    ygpu = H.f64(y[torch.as_tensor(rows, device=gpu)])
    err = H.max_rel_err(ygpu, yref)
    tol = H.TOL[cfg.expert_dtype if cfg.expert_dtype == "fp4" else cfg.act_dtype]
    print(f"[full] {name}: max rel err {err:.3e} (bar {tol})", flush=True)
    assert err <= tol
    # per-token bar too, so one bad token is not hidden by a large neighbour
    for i in range(rows.size):
        assert H.max_rel_err(ygpu[i:i + 1], yref[i:i + 1]) <= 2 * tol, f"token {rows[i]}"
    assert torch.isfinite(y.float()).all()
