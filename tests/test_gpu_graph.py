"""moe_forward and moe_forward_ex under HIP graph capture.  The forward does
no host synchronisation, allocation or memset, so a whole call can be
captured once and replayed.  The captured graph reads x from a fixed buffer,
so new inputs are copied into it before each replay.  Each case replays the
graph several times, with eager work and synchronisations between replays
and the input swapped in place, and checks every replay bit for bit against
an eager call on the same input."""

import pytest
import torch

from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu

CASES = [("tiny_fp32", False), ("v3_small", False), ("fp4_mx_small", False),
         ("fp4_mx_small", True), ("fp8_mx_small", True), ("hash_small", False)]


@pytest.mark.parametrize("name,side", CASES)
def test_graph_replays_match_eager(name, side, gpu):
    wl = C.SMALL_WORKLOADS[name]
    layer = synth.make_layer(wl, gpu)
    cfg, layer = H.run_weights(wl, wl.cfg, layer, B)
    if cfg.route_mode == "hash":
        table, _, _, _ = B.moe_build_tid2eid(layer["p"], cfg.n_routed_experts,
                                             cfg.n_activated_experts)
        layer["tid2eid"] = torch.from_numpy(table).to(gpu)
    T = wl.T
    inputs = [layer["x"].clone(), (torch.flip(layer["x"], dims=[0]) * -0.5).contiguous()]
    ws = B.alloc_workspace(cfg, T, gpu)
    side_stream = torch.cuda.Stream() if side else None

    def forward(x, y):
        if side:
            B.moe_forward_ex(cfg, layer, x, layer["token_ids"], T, y, ws, side_stream=side_stream)
        else:
            B.moe_forward(cfg, layer, x, layer["token_ids"], T, y, ws)

    refs = []
    for x in inputs:
        y = torch.empty_like(x)
        forward(x, y)
        torch.cuda.synchronize()
        refs.append(y.clone())
    assert not torch.equal(refs[0], refs[1])

    x_static = inputs[0].clone()
    y_static = torch.empty_like(x_static)
    forward(x_static, y_static)                      # warm up on the capture's buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"[graph] {name} side={side}: capture", flush=True)
    with torch.cuda.graph(g):
        forward(x_static, y_static)
    torch.cuda.synchronize()
    for r in range(4):
        i = r % 2
        x_static.copy_(inputs[i])
        y_static.fill_(float("nan"))                 # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] {name} side={side}: replay {r}", flush=True)
        assert torch.equal(y_static, refs[i]), f"replay {r} differs"
        scratch = (inputs[1 - i].float() * 2.0).sum()   # more eager work, then a sync
        torch.cuda.synchronize()
        del scratch
