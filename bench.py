#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward on one MI355X.

A step is one full forward of the layer (route -> permute -> grouped GEMM1
with SwiGLU -> grouped GEMM2 -> combine with the shared expert) over one
batch of synthetic tokens, through the C ABI (moe_forward_ex with stage
events and a second stream).  Inputs and weights are resident in HBM before
the timed region starts.  For FP4 / FP8 expert layers the library runs the
shared expert on the second stream during routing; the step time covers it
(the combine waits for it), the stage times do not.

Prints one JSON line:
  value        tokens/s of the DeepSeek-V3-shaped prefill layer (T=4096)
  roofline     the dominant kernel (grouped GEMM1: gate|up + SwiGLU; the
               routed experts' launch for FP4 / FP8 layers) against its
               bound, timed with HIP events on the library's stream
  cpu_baseline the float64 CPU oracle on a bounded sample of the same batch
  decode       the T=64 decode layer of the same weights (tokens/s, GB/s)
  graph_ms_per_step  the same step replayed from a captured HIP graph
  aux_ops      the path's other calls: selection-bias step, FP4 -> FP8
               re-dequantisation, host tid2eid builders (beside the oracle's)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at V3 shape (T=4096 prefill, T=64 decode) + % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
# sources of the grouped GEMM kernels a workload's GEMM1 runs on (a counter
# profile is only used while they are unchanged)
KERNEL_SOURCES = {
    "bf16": ("mixture_experts_ffn_route_amd/csrc/experts.hip",
             "mixture_experts_ffn_route_amd/csrc/gemm.h"),
    "mx": ("mixture_experts_ffn_route_amd/csrc/experts_mx.hip",
           "mixture_experts_ffn_route_amd/csrc/gemm.h"),
}


def gemm_kind(cfg):
    return "mx" if cfg.act_quant == "mxfp8" else "bf16"


def mfma_peak(cfg):
    """Dense MFMA peak of the dtype the expert contractions run in: FP8 x FP4
    scaled MFMA (FP8 rate) on MXFP8 activations, bf16 otherwise (FP4 experts
    on bf16 activations are decoded to bf16 in registers), fp32 for the fp32
    layer (plain FMA)."""
    if cfg.act_quant == "mxfp8":
        return MFMA_PEAK_TFLOPS["fp8"]
    return MFMA_PEAK_TFLOPS["f32" if cfg.act_dtype == "f32" else "bf16"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(kind="bf16"):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_counts(wl, counts):
    """Method work per step counted from the actual routing (intermediates
    such as H, Y and permuted copies are implementation traffic, excluded)."""
    cfg, T = wl.cfg, wl.T
    d, I, E, k = cfg.dim, cfg.moe_inter_dim, cfg.n_routed_experts, cfg.n_activated_experts
    eb = 4 if cfg.act_dtype == "f32" else 2
    if wl.fp8_weights:
        mat = I * d * (1.0 + 1.0 / 16384.0)       # E4M3 codes + one scale byte per 128x128
    elif cfg.expert_dtype == "fp4":
        mat = I * d * (0.5 + 1.0 / 32.0)          # codes + one scale byte per 32
    else:
        mat = I * d * eb
    n_hit = int((counts > 0).sum())
    sh = cfg.n_shared_experts
    rows = T * k + T * sh
    # the up-GEMM stage: FP4 / FP8 expert layers run the shared expert on the
    # second stream (moe_forward_ex), concurrently with the routing, outside the stage
    sh1 = 0 if (cfg.act_dtype == "bf16" and (cfg.expert_dtype == "fp4" or wl.fp8_weights)) else sh
    gemm1 = {"flops": 4.0 * d * I * (T * k + T * sh1),
             "bytes": n_hit * 2 * mat + sh1 * 2 * I * d * eb + T * d * eb}
    layer_flops = 6.0 * d * I * rows + (2.0 * T * d * E if cfg.route_mode == "learned" else 0.0)
    layer_bytes = n_hit * 3 * mat + sh * 3 * I * d * eb + 2 * T * d * eb
    layer_bytes += (E * d * eb + 4 * E) if cfg.route_mode == "learned" else 4 * T * k
    return {"n_hit": n_hit, "gemm1": gemm1, "layer": {"flops": layer_flops, "bytes": layer_bytes}}


def achievable_peaks(torch, B):
    """Achievable denominators on this GPU, from the library's roofline probes
    (the layer kernels' own instruction forms): 16-byte nontemporal loads streaming a
    4 GiB buffer, and chains of 16x16x32 bf16 MFMAs on every SIMD."""
    dev = torch.device("cuda:0")
    buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    out = torch.empty(4096, dtype=torch.int32, device=dev)
    for _ in range(2):
        B.moe_probe_read(buf, out)
        B.moe_probe_mfma(2000, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        B.moe_probe_read(buf, out)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    rates = {}
    for shape, name, iters in ((0, "16x16x32", 20000), (1, "32x32x16", 10000),
                               (2, "fp8xfp4 16x16x128", 2500), (3, "fp8xfp8 16x16x128", 2500)):
        B.moe_probe_mfma(10, out, shape)
        e0.record()
        flops = 0.0
        for _ in range(5):
            flops += B.moe_probe_mfma(iters, out, shape)
        e1.record()
        torch.cuda.synchronize()
        rates[name] = round(flops / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    del buf, out
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(read_gbs, 1),
            "bf16_mfma_tflops": max(rates["16x16x32"], rates["32x32x16"]),
            "fp8_mfma_tflops": max(rates["fp8xfp4 16x16x128"], rates["fp8xfp8 16x16x128"]),
            "mfma_tflops_by_shape": rates,
            "how": "moe_probe_read over 4 GiB; moe_probe_mfma (2048 x 4 waves; 8 independent "
                   "chains per wave for bf16, 16 for the scaled FP8 shapes)"}


def roofline_entry(flops, nbytes, seconds, peak_tflops):
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_mfma:
        ach = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    ach = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_tflops, "unit": "TFLOP/s",
            "frac": round(ach / peak_tflops, 4)}


def load_traffic(workload_name, kind="bf16"):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"grouped_gemm1_{workload_name}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def build_layer(wl, dev, B, synth):
    layer = synth.make_layer(wl, dev)
    if wl.cfg.route_mode == "hash":
        import torch
        table, _, _, _ = B.moe_build_tid2eid(layer["p"], wl.cfg.n_routed_experts,
                                             wl.cfg.n_activated_experts)
        layer["tid2eid"] = torch.from_numpy(table).to(dev)
    return layer


def run_weights(wl, layer, B, layout):
    """(config, layer) the timed steps use: the expert matrices rewritten once
    into the tiled layout (a load-time storage format) unless `layout` is
    "rows" or the layer is fp32; FP4 experts re-dequantised once to FP8 for
    the FP8-weight workloads (a load-time format too)."""
    if wl.fp8_weights:
        cfg8, layer8, lossy = B.redequant_layer(wl.cfg, layer)
        if lossy:
            log(f"{wl.name}: {lossy} lossy 128x128 blocks in the FP8 re-dequantisation")
        return cfg8, layer8
    if layout == "rows" or wl.cfg.act_dtype != "bf16":
        return wl.cfg, layer
    return B.pack_layer(wl.cfg, layer)


_SIDE_STREAM = None


def side_stream(torch):
    """The second stream moe_forward_ex gets, created once per process before
    any other (HIP spreads streams over a few hardware queues, four by
    default; a side stream that shares the main stream's queue runs in its
    order, not beside it, and every new stream is another draw)."""
    global _SIDE_STREAM
    if _SIDE_STREAM is None:
        _SIDE_STREAM = torch.cuda.Stream()
    return _SIDE_STREAM


def time_workload(wl, layer, steps, warmup, B, torch, cfg=None):
    cfg, T = (cfg or wl.cfg), wl.T
    dev = layer["x"].device
    ws = B.alloc_workspace(cfg, T, dev)
    y = torch.empty_like(layer["x"])
    nst = len(B.MOE_STAGES)
    ev = B.HipEvents((nst + 1) * steps)
    side = side_stream(torch)           # second stream for the work that needs x alone
    for _ in range(warmup):
        B.moe_forward_ex(cfg, layer, layer["x"], layer["token_ids"], T, y, ws, side_stream=side)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        B.moe_forward_ex(cfg, layer, layer["x"], layer["token_ids"], T, y, ws,
                         events=ev.handles[s * (nst + 1):(s + 1) * (nst + 1)], side_stream=side)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    stage_ms = {name: 0.0 for name in B.MOE_STAGES}
    for s in range(steps):
        base = s * (nst + 1)
        for i, name in enumerate(B.MOE_STAGES):
            stage_ms[name] += ev.elapsed_ms(base + i, base + i + 1) / steps
    ev.close()
    views = B.workspace_views(cfg, T, ws)
    counts = views["counts"].cpu().numpy()
    return total_ms / steps, stage_ms, counts


def time_graph(wl, layer, steps, B, torch, cfg=None):
    """ms per replay of one forward captured in a HIP graph (torch.cuda.CUDAGraph),
    the same call the timed steps make (second stream included): the launch
    overhead the eager steps pay is what the two numbers differ by."""
    cfg, T = (cfg or wl.cfg), wl.T
    ws = B.alloc_workspace(cfg, T, layer["x"].device)
    y = torch.empty_like(layer["x"])
    side = side_stream(torch)
    call = lambda: B.moe_forward_ex(cfg, layer, layer["x"], layer["token_ids"], T, y, ws,
                                    side_stream=side)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g, ws, y
    return ms


def workload_report(wl, ms, stage_ms, counts, peak):
    alg = algorithmic_counts(wl, counts)
    g1 = alg["gemm1"]
    roof = roofline_entry(g1["flops"], g1["bytes"], stage_ms["gemm1"] / 1e3, peak)
    lay = alg["layer"]
    layer_roof = roofline_entry(lay["flops"], lay["bytes"], ms / 1e3, peak)
    return {
        "tokens_per_s": round(wl.T / (ms / 1e3), 1),
        # both fractions of the whole layer step (the metric asks for MFMA and HBM %)
        "layer_mfma_frac": round(lay["flops"] / (ms / 1e3) / (peak * 1e12), 4),
        "layer_hbm_frac": round(lay["bytes"] / (ms / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
        "ms_per_step": round(ms, 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "experts_hit": alg["n_hit"],
        "gemm1": {**roof, "flops": g1["flops"], "bytes": g1["bytes"], "ms": round(stage_ms["gemm1"], 4)},
        "layer": {**layer_roof, "flops": lay["flops"], "bytes": lay["bytes"]},
    }


def aux_ops(torch, B, dev, synth, C):
    """The path's other calls, each on the shape it serves: the selection-bias
    step (V3: E=256), the load-time FP4 -> FP8 re-dequantisation (the
    V4.1-Flash gate|up matrices, 384 x 1536 x 5120), and the host tid2eid
    builders (m=32768 Zipf(1.1), n=64, k=4; greedy and an 8-order multi-start),
    the last two beside the oracle's own time."""
    import numpy as np
    import oracle
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    cfg = C.V3_PREFILL.cfg
    E, k, T = cfg.n_routed_experts, cfg.n_activated_experts, C.V3_PREFILL.T
    g = torch.Generator(device="cpu").manual_seed(7)
    counts = torch.randint(64, 200, (E,), generator=g, dtype=torch.int32).to(dev)
    bias = torch.zeros(E, dtype=torch.float32, device=dev)
    stats = torch.zeros(4, dtype=torch.float64, device=dev)
    for _ in range(10):
        B.moe_update_bias(cfg, counts, T, 1e-3, bias, stats)
    torch.cuda.synchronize()
    n = 200
    e0.record()
    for _ in range(n):
        B.moe_update_bias(cfg, counts, T, 1e-3, bias, stats)
    e1.record()
    torch.cuda.synchronize()
    out["update_bias"] = {"E": E, "us_per_call": round(e0.elapsed_time(e1) / n * 1e3, 2),
                          "bound": "latency (one small workgroup)"}

    n_mat, N, K = 384, 1536, 5120
    codes = torch.randint(0, 256, (n_mat, N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.randint(118, 127, (n_mat, N, K // 32), dtype=torch.uint8, device=dev)
    fp8 = torch.empty(n_mat * N * K, dtype=torch.uint8, device=dev)
    bsc = torch.empty((n_mat, N // 128, K // 128), dtype=torch.uint8, device=dev)
    lossy = torch.empty_like(bsc)
    B.moe_redequant_fp8(codes, scales, n_mat, N, K, fp8, bsc, lossy)
    torch.cuda.synchronize()
    n = 5
    e0.record()
    for _ in range(n):
        B.moe_redequant_fp8(codes, scales, n_mat, N, K, fp8, bsc, lossy)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = codes.numel() + scales.numel() + fp8.numel() + 2 * bsc.numel()
    out["redequant_fp8"] = {"shape": [n_mat, N, K], "ms": round(ms, 4),
                            **roofline_entry(0.0, nbytes, ms / 1e3, 1.0), "bytes": nbytes}
    del codes, scales, fp8, bsc, lossy
    torch.cuda.empty_cache()

    p = synth.zipf_probs(32768, 1.1)
    rng = np.random.default_rng(3)
    orders = np.stack([rng.permutation(p.shape[0]) for _ in range(8)])
    t = time.perf_counter()
    B.moe_build_tid2eid(p, 64, 4)
    lib_ms = (time.perf_counter() - t) * 1e3
    t = time.perf_counter()
    B.moe_build_tid2eid_multistart(p, 64, 4, orders)
    lib_ms8 = (time.perf_counter() - t) * 1e3
    t = time.perf_counter()
    oracle.tid2eid_greedy(p, 64, 4)
    ora_ms = (time.perf_counter() - t) * 1e3
    out["tid2eid_host"] = {"m": int(p.shape[0]), "n": 64, "k": 4, "greedy_ms": round(lib_ms, 2),
                           "multistart_8_ms": round(lib_ms8, 2),
                           "oracle_greedy_ms": round(ora_ms, 2), "threads": 1}
    return out


# Tokens of each workload the CPU oracle is timed on: whole batches where the
# oracle finishes them in seconds (the fp32 layer, the T=64 decode batch, the
# hash layers), else the first tokens of the batch (the oracle's cost is the
# experts those tokens touch, each widened to float64 at use).
CPU_SAMPLE = {"tiny_fp32": None, "v3_decode": None, "hash_bf16": None, "ngram_bf16": None,
              "v3_prefill": 96, "v41_flash_fp4": 16, "v41_flash_fp4_mx": 16,
              "v41_flash_fp8": 8}


def cpu_baseline(wl, layer, sample_tokens=None):
    """The float64 oracle, as it is, on the first `sample_tokens` tokens (all
    when None): routing + permutation + routed/shared SwiGLU forward (MXFP8
    activations for the MXFP8 layers).  The experts the sample touches are
    staged on the host in their stored format first (untimed; for the
    FP8-weight layer that format is the oracle's own FP4 -> FP8
    re-dequantisation, a load-time conversion like the GPU's, run in worker
    processes); their widening to float64 is the oracle's work and is timed."""
    import numpy as np
    import torch
    import oracle
    from threadpoolctl import threadpool_info

    cfg = wl.cfg
    S = wl.T if sample_tokens is None else min(sample_tokens, wl.T)
    f32 = lambda t: t.detach().float().cpu().numpy()
    x = f32(layer["x"][:S])
    ids = None if layer.get("token_ids") is None else layer["token_ids"][:S].cpu().numpy()
    table = None
    if cfg.route_mode == "hash":
        table, _, _, _ = oracle.tid2eid_greedy(layer["p"], cfg.n_routed_experts,
                                               cfg.n_activated_experts)
    bias = None if layer.get("gate_bias") is None else layer["gate_bias"].cpu().numpy()
    gate_w = f32(layer["gate_w"]) if cfg.route_mode == "learned" else None

    def route():
        if cfg.route_mode == "hash":
            return oracle.hash_gate(ids, table, cfg.route_scale)
        if cfg.route_mode == "ngram":
            return oracle.ngram_hash_gate(ids[:, 0], ids[:, 1], cfg.vocab_size,
                                          cfg.n_routed_experts, cfg.n_activated_experts,
                                          cfg.route_scale)
        w, i, _ = oracle.learned_gate(x, gate_w, bias, score_func=cfg.score_func,
                                      n_groups=cfg.n_expert_groups,
                                      topk_groups=cfg.n_limited_groups,
                                      topk=cfg.n_activated_experts, route_scale=cfg.route_scale,
                                      renormalize=cfg.renormalize)
        return w, i

    _, idx = route()
    mats = ("w_gate", "w_up", "w_down")
    host = {}
    touched = [int(e) for e in np.unique(idx)]
    if wl.fp8_weights:
        import multiprocessing
        from concurrent.futures import ProcessPoolExecutor
        with ProcessPoolExecutor(16, mp_context=multiprocessing.get_context("spawn")) as pool:
            futs = {e: [pool.submit(oracle.fp4_to_fp8_blocks, layer[n][e].cpu().numpy(),
                                    layer["s_" + n[2:]][e].cpu().numpy()) for n in mats]
                    for e in touched}
            for e in touched:
                host[e] = tuple(f.result()[:2] for f in futs[e])
    elif cfg.expert_dtype == "fp4":
        for e in touched:
            host[e] = tuple((layer[n][e].cpu().numpy(), layer["s_" + n[2:]][e].cpu().numpy())
                            for n in mats)
    else:
        for e in touched:
            host[e] = tuple(layer[n][e].cpu() for n in mats)
    shared_host = None
    if cfg.n_shared_experts:
        shared_host = tuple(layer[n].cpu() for n in ("sh_gate", "sh_up", "sh_down"))

    def expert(e):
        if wl.fp8_weights:
            return tuple(oracle.fp8_blocks_decode(c, b) for c, b in host[e])
        if cfg.expert_dtype == "fp4":
            return tuple(oracle.fp4_decode(p, s) for p, s in host[e])
        return tuple(a.double().numpy() for a in host[e])

    forward = oracle.layer_forward_mx if cfg.act_quant == "mxfp8" else oracle.layer_forward
    t0 = time.perf_counter()
    w, idx = route()
    oracle.permute(idx, cfg.n_routed_experts)
    shared = None
    if shared_host is not None:
        shared = tuple(a.double().numpy() for a in shared_host)
    forward(x, w, idx, expert, shared, cfg.swiglu_limit)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [torch.get_num_threads()])
    what = "all" if S == wl.T else f"the first {S} of the"
    return {"value": round(S / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} {wl.T} tokens of {wl.name}: route + permute + routed and shared "
                      f"SwiGLU in float64 ({len(host)} experts touched), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--decode", default="v3_decode", help="second workload ('' to skip)")
    ap.add_argument("--extra", default="hash_bf16,ngram_bf16,v41_flash_fp4,v41_flash_fp4_mx,"
                                      "v41_flash_fp8,tiny_fp32",
                    help="comma-separated further workloads to report ('' for none)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=CPU_SAMPLE["v3_prefill"],
                    help="tokens of the headline batch the CPU oracle is timed on (about 10 s); "
                         "the other workloads use their CPU_SAMPLE entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable matmul / HBM-read denominators and "
                         "timing the auxiliary calls (bias step, FP8 re-dequantisation, "
                         "tid2eid builders)")
    ap.add_argument("--layout", choices=("tiled", "rows"), default="tiled",
                    help="expert weight storage the timed steps read (tiled: packed once by "
                         "moe_pack_weights before timing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: every box here has one MI355X and this layer "
              f"holds all experts on one GPU (asked for --gpus {args.gpus}, WORLD_SIZE={world})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_ffn_route_amd import binding as B
    from mixture_experts_ffn_route_amd import config as C
    from mixture_experts_ffn_route_amd import synth

    dev = torch.device("cuda:0")
    side_stream(torch)                  # before any other stream (see side_stream)
    wl = C.FULL_WORKLOADS[args.workload]
    log(f"generating {wl.name} inputs on {torch.cuda.get_device_name(0)}")
    t = time.time()
    layer = build_layer(wl, dev, B, synth)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t:.1f} s; timing {args.steps} steps after {args.warmup} warmup")
    peak = mfma_peak(wl.cfg)
    rcfg, rlayer = run_weights(wl, layer, B, args.layout)
    torch.cuda.synchronize()
    ms, stage_ms, counts = time_workload(wl, rlayer, args.steps, args.warmup, B, torch, rcfg)
    rep = workload_report(wl, ms, stage_ms, counts, peak)
    log(f"{wl.name}: {rep['ms_per_step']} ms/step, {rep['tokens_per_s']} tokens/s, stages {rep['stage_ms']}")

    out = {
        "metric": METRIC,
        "value": rep["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rep["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4" if wl.cfg.expert_dtype == "fp4" else wl.cfg.act_dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "dim": wl.cfg.dim,
                   "n_routed_experts": wl.cfg.n_routed_experts,
                   "n_activated_experts": wl.cfg.n_activated_experts,
                   "moe_inter_dim": wl.cfg.moe_inter_dim,
                   "n_shared_experts": wl.cfg.n_shared_experts,
                   "weight_layout": rcfg.weight_layout,
                   "parallelism": "single-gpu (all experts resident)"},
    }
    g1 = rep["gemm1"]
    out["roofline"] = {"kernel": "grouped_gemm1 (gate|up + SwiGLU)", "bound": g1["bound"],
                       "achieved": g1["achieved"], "peak": g1["peak"], "unit": g1["unit"],
                       "frac": g1["frac"], "traffic": load_traffic(wl.name, gemm_kind(wl.cfg)),
                       "algorithmic_bytes": g1["bytes"], "algorithmic_flops": g1["flops"],
                       "avg_ms": g1["ms"]}
    out["layer_roofline"] = {**rep["layer"], "mfma_frac": rep["layer_mfma_frac"],
                             "hbm_frac": rep["layer_hbm_frac"]}
    out["stage_ms"] = rep["stage_ms"]
    out["graph_ms_per_step"] = round(time_graph(wl, rlayer, args.steps, B, torch, rcfg), 4)

    reports = {}
    names = ([args.decode] if args.decode else []) + [n for n in args.extra.split(",") if n]
    for name in names:
        w2 = C.FULL_WORKLOADS[name]
        if (w2.cfg == wl.cfg and w2.seed == wl.seed and w2.fp8_weights == wl.fp8_weights
                and max(w2.T, w2.x_rows) == wl.T):
            # same layer and weights; x is the first T rows of the same draw
            l2 = dict(rlayer)
            l2["x"] = layer["x"][:w2.T].contiguous()
            c2cfg = rcfg
            l2_src = dict(layer, x=l2["x"])
        else:
            log(f"generating {name} inputs")
            l2_src = build_layer(w2, dev, B, synth)
            c2cfg, l2 = run_weights(w2, l2_src, B, args.layout)
        p2 = mfma_peak(w2.cfg)
        ms2, st2, c2 = time_workload(w2, l2, args.steps, args.warmup, B, torch, c2cfg)
        r2 = workload_report(w2, ms2, st2, c2, p2)
        r2["graph_ms_per_step"] = round(time_graph(w2, l2, args.steps, B, torch, c2cfg), 4)
        r2["roofline"] = {k: r2["gemm1"][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
        r2["roofline"]["traffic"] = load_traffic(name, gemm_kind(w2.cfg))
        if not args.no_cpu_baseline:
            log(f"{name}: timing the CPU oracle")
            r2["cpu_baseline"] = cpu_baseline(w2, l2_src, CPU_SAMPLE.get(name, 16))
            log(f"{name}: cpu_baseline {r2['cpu_baseline']}")
        reports[name] = r2
        log(f"{name}: {r2['ms_per_step']} ms/step (graph {r2['graph_ms_per_step']}), {r2['tokens_per_s']} tokens/s, stages {r2['stage_ms']}")
        del l2, l2_src
    if args.decode:
        out["decode"] = {"workload": args.decode, **reports.pop(args.decode)}
    if reports:
        out["extra_workloads"] = reports

    if not args.no_peaks:
        log("measuring achievable peaks")
        pk = achievable_peaks(torch, B)
        out["achievable_peaks"] = pk
        r = out["roofline"]
        denom = pk["hbm_read_gbs"] if r["unit"] == "GB/s" else pk["bf16_mfma_tflops"]
        r["frac_of_achievable"] = round(r["achieved"] / denom, 4)
        for rep in [out.get("decode")] + list((out.get("extra_workloads") or {}).values()):
            if not rep:
                continue
            rr = rep["roofline"]
            if rr["unit"] == "GB/s":
                rr["frac_of_achievable"] = round(rr["achieved"] / pk["hbm_read_gbs"], 4)
            else:
                key = {MFMA_PEAK_TFLOPS["fp8"]: "fp8_mfma_tflops",
                       MFMA_PEAK_TFLOPS["bf16"]: "bf16_mfma_tflops"}.get(rr["peak"])
                if key:
                    rr["frac_of_achievable"] = round(rr["achieved"] / pk[key], 4)
        log(f"achievable: {pk}")
    if not args.no_peaks:
        log("timing the auxiliary calls")
        out["aux_ops"] = aux_ops(torch, B, dev, synth, C)
        log(f"aux: {out['aux_ops']}")
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_sample_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(wl, layer, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
