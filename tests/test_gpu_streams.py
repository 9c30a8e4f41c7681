"""Stream ordering of moe_forward.  FP4 / FP8 expert layers run the shared
expert and the MXFP8 copy of x on a library side stream forked from the
caller's stream and joined before the combine; these tests check that the
fork and join order the work correctly.  Every result must equal a lone
call on the default stream bit for bit, because the layer is deterministic.
The cases are: a call on a non-default stream, back-to-back calls that reuse
one workspace with different inputs, and two host threads calling at once on
streams of their own.  The accuracy bar against the oracle is the parity
tests' job; bf16 expert layers, which use no side stream, are included as a
control."""

import threading

import pytest
import torch

from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu

NAMES = ["fp4_mx_small", "fp8_mx_small", "fp4_small", "v3_small"]


def _setup(name, dev):
    wl = C.SMALL_WORKLOADS[name]
    layer = synth.make_layer(wl, dev)
    cfg, layer = H.run_weights(wl, wl.cfg, layer, B)
    x2 = torch.flip(layer["x"], dims=[0]) * -0.75          # a second input of the same shape
    torch.cuda.synchronize()
    return wl, cfg, layer, x2


def _forward(cfg, layer, x, T, ws, stream=None):
    y = torch.empty_like(x)
    B.moe_forward(cfg, layer, x, layer["token_ids"], T, y, ws, stream=stream)
    return y


def _lone(cfg, layer, x, T, dev):
    ws = B.alloc_workspace(cfg, T, dev)
    y = _forward(cfg, layer, x, T, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", NAMES)
def test_non_default_stream(name, gpu):
    wl, cfg, layer, _ = _setup(name, gpu)
    ref = _lone(cfg, layer, layer["x"], wl.T, gpu)
    ws = B.alloc_workspace(cfg, wl.T, gpu)
    y = torch.empty_like(layer["x"])
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    print(f"[streams] {name}: forward on a non-default stream", flush=True)
    B.moe_forward(cfg, layer, layer["x"], layer["token_ids"], wl.T, y, ws, stream=s)
    s.synchronize()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("name", NAMES)
def test_back_to_back_calls_reuse_one_workspace(name, gpu):
    wl, cfg, layer, x2 = _setup(name, gpu)
    ref1 = _lone(cfg, layer, layer["x"], wl.T, gpu)
    ref2 = _lone(cfg, layer, x2, wl.T, gpu)
    assert not torch.equal(ref1, ref2)
    ws = B.alloc_workspace(cfg, wl.T, gpu)
    print(f"[streams] {name}: 4 back-to-back calls on one workspace", flush=True)
    ys = [_forward(cfg, layer, x, wl.T, ws) for x in (layer["x"], x2, layer["x"], x2)]
    torch.cuda.synchronize()
    for y, ref in zip(ys, (ref1, ref2, ref1, ref2)):
        assert torch.equal(y, ref)


@pytest.mark.parametrize("name", ["fp4_mx_small", "v3_small"])
def test_two_host_threads(name, gpu):
    wl, cfg, layer, x2 = _setup(name, gpu)
    refs = [_lone(cfg, layer, layer["x"], wl.T, gpu), _lone(cfg, layer, x2, wl.T, gpu)]
    inputs = [layer["x"], x2]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [B.alloc_workspace(cfg, wl.T, gpu) for _ in range(2)]
    outs = [[torch.empty_like(layer["x"]) for _ in range(6)] for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(gpu)
            for j, y in enumerate(outs[i]):
                B.moe_forward(cfg, layer, inputs[(i + j) % 2], layer["token_ids"], wl.T, y,
                              wss[i], stream=streams[i])
            streams[i].synchronize()
        except Exception as e:                # reported by the main thread
            errors.append(e)

    print(f"[streams] {name}: two host threads, 6 calls each", flush=True)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for i in range(2):
        for j, y in enumerate(outs[i]):
            assert torch.equal(y, refs[(i + j) % 2]), (i, j)
