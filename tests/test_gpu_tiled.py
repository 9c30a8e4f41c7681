"""GPU tests of the tiled weight layout (moe_pack_weights).

The packed bytes are checked against the layout written out with numpy
reshapes (tiles of 16 outputs x 32 bf16 inputs / 64 FP4 inputs, each lane's
group of consecutive inputs contiguous), and moe_forward on tiled weights must
give bit-identical outputs to the row layout, whose parity with the oracle the
other GPU tests establish.
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


def _tiled_bf16(w):
    """[E, N, K] -> tiled order: (E, N/16, K/32, K%32 // 8, N%16, K%8)."""
    E, N, K = w.shape
    return w.reshape(E, N // 16, 16, K // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(E, N, K)


def _tiled_fp4_codes(q):
    """bytes [E, N, K/2] -> (E, N/16, K/64, byte%32 // 8, N%16, byte%8)."""
    E, N, KB = q.shape
    return q.reshape(E, N // 16, 16, KB // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(E, N, KB)


def _tiled_scales(s):
    """[E, N, K/32] -> (E, N/16, K/64, N%16, block%2)."""
    E, N, KS = s.shape
    return s.reshape(E, N // 16, 16, KS // 2, 2).transpose(0, 1, 3, 2, 4).reshape(E, N, KS)


def _u16(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("name", ["v3_small", "fp4_small", "fp4_odd_widths"])
def test_pack_layout(name, gpu):
    wl = C.SMALL_WORKLOADS[name]
    cfg = wl.cfg
    layer = synth.make_layer(wl, gpu)
    print(f"[pack] {name}", flush=True)
    tcfg, packed = B.pack_layer(cfg, layer)
    torch.cuda.synchronize()
    assert tcfg.weight_layout == "tiled"
    for n in ("w_gate", "w_up", "w_down"):
        src, dst = layer[n], packed[n]
        if cfg.expert_dtype == "fp4":
            np.testing.assert_array_equal(dst.cpu().numpy(), _tiled_fp4_codes(src.cpu().numpy()))
            s = "s_" + n[2:]
            np.testing.assert_array_equal(packed[s].cpu().numpy(),
                                          _tiled_scales(layer[s].cpu().numpy()))
        else:
            np.testing.assert_array_equal(_u16(dst), _tiled_bf16(_u16(src)))
    for n in ("sh_gate", "sh_up", "sh_down"):
        np.testing.assert_array_equal(_u16(packed[n])[None], _tiled_bf16(_u16(layer[n])[None]))
    # members that are not expert matrices are shared, not copied
    assert packed["gate_w"] is layer["gate_w"]


def _forward(cfg, layer, T, device, with_ws=False):
    ws = B.alloc_workspace(cfg, T, device)
    y = torch.empty_like(layer["x"])
    B.moe_forward(cfg, layer, layer["x"], layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    return (y, ws) if with_ws else y


@pytest.mark.parametrize("name", [n for n, w in C.SMALL_WORKLOADS.items()
                                  if w.cfg.act_dtype == "bf16"])
def test_forward_tiled_equals_rows(name, gpu):
    wl = C.SMALL_WORKLOADS[name]
    cfg, T = wl.cfg, wl.T
    layer = synth.make_layer(wl, gpu)
    if cfg.route_mode == "hash":
        table, _, _, _ = B.moe_build_tid2eid(layer["p"], cfg.n_routed_experts,
                                             cfg.n_activated_experts)
        layer["tid2eid"] = torch.from_numpy(table).to(gpu)
    print(f"[tiled] {name}", flush=True)
    y_rows = _forward(cfg, layer, T, gpu)
    tcfg, packed = B.pack_layer(cfg, layer)
    y_tiled = _forward(tcfg, packed, T, gpu)
    assert torch.equal(y_rows.view(torch.int16), y_tiled.view(torch.int16))
    assert torch.isfinite(y_tiled.float()).all()


def test_forward_tiled_decode_and_single_token(gpu):
    """Tile heights 1 and 4 row blocks (decode configurations) on tiled weights."""
    wl = C.SMALL_WORKLOADS["v3_decode_small"]
    cfg = wl.cfg
    layer = synth.make_layer(wl, gpu)
    tcfg, packed = B.pack_layer(cfg, layer)
    for T in (1, 5, 13):
        print(f"[tiled] decode T={T}", flush=True)
        sub = dict(layer, x=layer["x"][:T].contiguous())
        psub = dict(packed, x=sub["x"])
        y_rows = _forward(cfg, sub, T, gpu)
        y_tiled, ws = _forward(tcfg, psub, T, gpu, with_ws=True)
        assert torch.equal(y_rows.view(torch.int16), y_tiled.view(torch.int16))
        v = B.workspace_views(cfg, T, ws)
        ow, oidx, aux = H.oracle_route(cfg, sub)
        rc = H.check_routing(cfg, H.cpu_np(v["route_weights"]), H.cpu_np(v["route_indices"]),
                             ow, oidx, aux, label=f"decode T={T}")
        yref = oracle.layer_forward(H.f64(sub["x"]), rc.ref_w, rc.idx,
                                    H.expert_fetcher(layer, cfg), H.shared_weights(layer, cfg),
                                    cfg.swiglu_limit)
        H.check_layer_output(cfg, H.f64(y_tiled), yref, label=f"decode T={T}")
