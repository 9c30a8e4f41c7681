"""Stream ordering of moe_forward_ex with a second stream.  FP4 / FP8 expert
layers then run the shared expert and the MXFP8 copy of x on the caller's
side stream, forked from the main stream and joined before the combine;
these tests check that the fork and join order the work correctly.  Every
result must equal moe_forward's on the default stream bit for bit, because
the layer is deterministic and both paths run the same kernels in the same
order per output.  The cases are: a call on non-default streams, back-to-back
calls that reuse one workspace with different inputs, and two host threads
calling at once on streams of their own.  The accuracy bar against the oracle
is the parity tests' job; bf16 expert layers, which ignore the side stream,
are included as a control."""

import threading

import pytest
import torch

from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu

# fp4_odd_widths: shared widths that are not multiples of 128 (the shared gate|up
# on the grouped kernel's dense form); *_decode: one-row-block tiles
NAMES = ["fp4_mx_small", "fp8_mx_small", "fp4_small", "fp4_odd_widths", "fp4_mx_decode",
         "fp8_mx_decode", "v3_small"]


def _setup(name, dev):
    wl = C.SMALL_WORKLOADS[name]
    layer = synth.make_layer(wl, dev)
    cfg, layer = H.run_weights(wl, wl.cfg, layer, B)
    x2 = torch.flip(layer["x"], dims=[0]) * -0.75          # a second input of the same shape
    torch.cuda.synchronize()
    return wl, cfg, layer, x2


def _lone(cfg, layer, x, T, dev):
    """moe_forward (one stream) on the default stream."""
    ws = B.alloc_workspace(cfg, T, dev)
    y = torch.empty_like(x)
    B.moe_forward(cfg, layer, x, layer["token_ids"], T, y, ws)
    torch.cuda.synchronize()
    return y


def _forward_ex(cfg, layer, x, T, ws, y, stream, side):
    B.moe_forward_ex(cfg, layer, x, layer["token_ids"], T, y, ws, stream=stream,
                     side_stream=side)


@pytest.mark.parametrize("name", NAMES)
def test_side_stream_matches_one_stream(name, gpu):
    wl, cfg, layer, _ = _setup(name, gpu)
    ref = _lone(cfg, layer, layer["x"], wl.T, gpu)
    ws = B.alloc_workspace(cfg, wl.T, gpu)
    y = torch.empty_like(layer["x"])
    torch.cuda.synchronize()
    s, side = torch.cuda.Stream(), torch.cuda.Stream()
    print(f"[streams] {name}: moe_forward_ex on two non-default streams", flush=True)
    _forward_ex(cfg, layer, layer["x"], wl.T, ws, y, s, side)
    s.synchronize()
    assert torch.equal(y, ref)


@pytest.mark.parametrize("name", NAMES)
def test_back_to_back_calls_reuse_one_workspace(name, gpu):
    wl, cfg, layer, x2 = _setup(name, gpu)
    ref1 = _lone(cfg, layer, layer["x"], wl.T, gpu)
    ref2 = _lone(cfg, layer, x2, wl.T, gpu)
    assert not torch.equal(ref1, ref2)
    ws = B.alloc_workspace(cfg, wl.T, gpu)
    ys = [torch.empty_like(layer["x"]) for _ in range(4)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    print(f"[streams] {name}: 4 back-to-back calls on one workspace", flush=True)
    for x, y in zip((layer["x"], x2, layer["x"], x2), ys):
        _forward_ex(cfg, layer, x, wl.T, ws, y, torch.cuda.current_stream(), side)
    torch.cuda.synchronize()
    for y, ref in zip(ys, (ref1, ref2, ref1, ref2)):
        assert torch.equal(y, ref)


@pytest.mark.parametrize("name", ["fp4_mx_small", "v3_small"])
def test_two_host_threads(name, gpu):
    wl, cfg, layer, x2 = _setup(name, gpu)
    refs = [_lone(cfg, layer, layer["x"], wl.T, gpu), _lone(cfg, layer, x2, wl.T, gpu)]
    inputs = [layer["x"], x2]
    streams = [(torch.cuda.Stream(), torch.cuda.Stream()) for _ in range(2)]
    wss = [B.alloc_workspace(cfg, wl.T, gpu) for _ in range(2)]
    outs = [[torch.empty_like(layer["x"]) for _ in range(6)] for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(gpu)
            for j, y in enumerate(outs[i]):
                _forward_ex(cfg, layer, inputs[(i + j) % 2], wl.T, wss[i], y, *streams[i])
            streams[i][0].synchronize()
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


@pytest.mark.parametrize("name", ["fp4_mx_small", "v3_small"])
def test_stage_events_with_side_stream(name, gpu):
    """moe_forward_ex with stage events and a side stream: the same output, and
    every stage interval recorded (non-negative, summing to at most the call)."""
    wl, cfg, layer, _ = _setup(name, gpu)
    ref = _lone(cfg, layer, layer["x"], wl.T, gpu)
    ws = B.alloc_workspace(cfg, wl.T, gpu)
    y = torch.empty_like(layer["x"])
    nst = len(B.MOE_STAGES)
    ev = B.HipEvents(nst + 1)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    print(f"[streams] {name}: moe_forward_ex with stage events", flush=True)
    B.moe_forward_ex(cfg, layer, layer["x"], layer["token_ids"], wl.T, y, ws, events=ev.handles,
                     side_stream=side)
    torch.cuda.synchronize()
    stages = [ev.elapsed_ms(i, i + 1) for i in range(nst)]
    total = ev.elapsed_ms(0, nst)
    ev.close()
    assert torch.equal(y, ref)
    assert all(s >= 0.0 for s in stages) and sum(stages) <= total * 1.001 + 1e-3
