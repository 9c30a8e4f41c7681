"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, validates arguments on the host, and its host-only
tid2eid builder agrees with the oracle bit for bit."""

import ctypes
import os
import re
import subprocess
from dataclasses import replace

import numpy as np
import pytest

import oracle
from mixture_experts_ffn_route_amd import binding as B
from mixture_experts_ffn_route_amd import config as C
from mixture_experts_ffn_route_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(B.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)$", out, re.M))
    assert set(declared_functions()) <= exported


def test_status_strings():
    assert B.moe_status_string(0) == "MOE_OK"
    assert B.moe_status_string(-1) == "MOE_ERR_INVALID_ARG"
    assert B.moe_status_string(-3) == "MOE_ERR_WORKSPACE"
    assert B.moe_status_string(123) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("name", list(C.FULL_WORKLOADS) + list(C.SMALL_WORKLOADS))
def test_named_workloads_are_valid(name):
    wl = {**C.FULL_WORKLOADS, **C.SMALL_WORKLOADS}[name]
    assert B.moe_validate_config(wl.cfg) == B.MOE_OK


V3 = C.V3_PREFILL.cfg
BAD = [
    ("E % G", replace(V3, n_expert_groups=7), B.MOE_ERR_INVALID_ARG),
    ("k > E", replace(V3, n_routed_experts=4, n_expert_groups=1, n_limited_groups=1), B.MOE_ERR_INVALID_ARG),
    ("kept groups > G", replace(V3, n_limited_groups=9), B.MOE_ERR_INVALID_ARG),
    ("k > kept experts", replace(V3, n_limited_groups=1, n_activated_experts=33), B.MOE_ERR_INVALID_ARG),
    ("zero dim", replace(V3, dim=0), B.MOE_ERR_INVALID_ARG),
    ("negative clamp", replace(V3, swiglu_limit=-1.0), B.MOE_ERR_INVALID_ARG),
    ("bad renormalize", replace(V3, renormalize=2), B.MOE_ERR_INVALID_ARG),
    ("fp32 act with bf16 experts", replace(V3, act_dtype="f32"), B.MOE_ERR_INVALID_ARG),
    ("hash without vocab", replace(C.HASH_BF16.cfg, vocab_size=0), B.MOE_ERR_INVALID_ARG),
    ("bf16 dim % 64", replace(V3, dim=7168 + 32), B.MOE_ERR_UNSUPPORTED),
    ("fp4 dim % 64", replace(C.V41_FLASH_FP4.cfg, dim=5120 + 32), B.MOE_ERR_UNSUPPORTED),
    ("two shared experts", replace(V3, n_shared_experts=2), B.MOE_ERR_UNSUPPORTED),
    ("k > 16", replace(V3, n_activated_experts=17, n_limited_groups=8), B.MOE_ERR_UNSUPPORTED),
    ("learned E > 512", replace(V3, n_routed_experts=1024, n_expert_groups=1, n_limited_groups=1), B.MOE_ERR_UNSUPPORTED),
    ("group lanes not a power of two", replace(V3, n_routed_experts=96, n_expert_groups=8, n_limited_groups=4), B.MOE_ERR_UNSUPPORTED),
    ("tiled fp32 layer", replace(C.TINY_FP32.cfg, weight_layout="tiled"), B.MOE_ERR_UNSUPPORTED),
    ("mxfp8 on bf16 experts", replace(V3, act_quant="mxfp8"), B.MOE_ERR_INVALID_ARG),
    ("mxfp8 dim % 128", replace(C.V41_FLASH_FP4_MX.cfg, dim=5120 + 64), B.MOE_ERR_UNSUPPORTED),
    ("mxfp8 inter % 128", replace(C.V41_FLASH_FP4_MX.cfg, moe_inter_dim=1536 + 64), B.MOE_ERR_UNSUPPORTED),
    ("fp8 experts on bf16 activations", replace(C.V41_FLASH_FP4.cfg, expert_dtype="fp8", weight_layout="tiled"), B.MOE_ERR_INVALID_ARG),
    ("fp8 experts in the row layout", replace(C.V41_FLASH_FP4_MX.cfg, expert_dtype="fp8"), B.MOE_ERR_INVALID_ARG),
    ("fp8 experts, dim > 32768", replace(C.V41_FLASH_FP4_MX.cfg, expert_dtype="fp8", weight_layout="tiled", dim=32768 + 128), B.MOE_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("what,cfg,status", BAD, ids=[b[0] for b in BAD])
def test_validation_errors(what, cfg, status):
    assert B.moe_validate_config(cfg) == status
    assert B.moe_workspace_size(cfg, 16) == 0


def test_enum_range_checked():
    c = B.config_c(V3)
    c.score_func = 3
    assert B._lib.moe_validate_config(ctypes.byref(c)) == B.MOE_ERR_INVALID_ARG
    c = B.config_c(V3)
    c.route_mode = 2
    assert B._lib.moe_validate_config(ctypes.byref(c)) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_validate_config(None) == B.MOE_ERR_INVALID_ARG
    c = B.config_c(V3)
    c.weight_layout = 2
    assert B._lib.moe_validate_config(ctypes.byref(c)) == B.MOE_ERR_INVALID_ARG
    c = B.config_c(C.V41_FLASH_FP4.cfg)
    c.act_quant = 2
    assert B._lib.moe_validate_config(ctypes.byref(c)) == B.MOE_ERR_INVALID_ARG
    assert B.moe_validate_config(replace(V3, weight_layout="tiled")) == B.MOE_OK


def test_pack_rejects_before_any_launch():
    """moe_pack_weights checks its arguments on the host: null structs, a set
    source member without a destination, in-place packing, fp32 layers."""
    fake, other = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000)
    cc = B.config_c(V3)
    full = B.MoeWeightsC(*([fake] * 12))
    pack = B._lib.moe_pack_weights
    assert pack(None, ctypes.byref(full), ctypes.byref(full), None) == B.MOE_ERR_INVALID_ARG
    assert pack(ctypes.byref(cc), None, ctypes.byref(full), None) == B.MOE_ERR_INVALID_ARG
    assert pack(ctypes.byref(cc), ctypes.byref(full), None, None) == B.MOE_ERR_INVALID_ARG
    assert pack(ctypes.byref(cc), ctypes.byref(full), ctypes.byref(full), None) == B.MOE_ERR_INVALID_ARG
    dst = B.MoeWeightsC(*([other] * 12))
    dst.w_up = None
    assert pack(ctypes.byref(cc), ctypes.byref(full), ctypes.byref(dst), None) == B.MOE_ERR_INVALID_ARG
    f32 = B.config_c(C.TINY_FP32.cfg)
    assert pack(ctypes.byref(f32), ctypes.byref(full), ctypes.byref(B.MoeWeightsC(*([other] * 12))),
                None) == B.MOE_ERR_INVALID_ARG
    bad = B.config_c(replace(V3, dim=7168 + 32))
    assert pack(ctypes.byref(bad), ctypes.byref(full), ctypes.byref(B.MoeWeightsC(*([other] * 12))),
                None) == B.MOE_ERR_UNSUPPORTED


def test_forward_rejects_before_any_launch():
    """Host validation returns before touching the device: null workspace,
    too-small workspace, null pointers, aliasing x and y."""
    cfg = C.SMALL_WORKLOADS["v3_small"].cfg
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: validation fails first
    layer = {n: None for n in ("gate_w", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")}
    wc = B.weights_c(layer)
    cc = B.config_c(cfg)
    st = B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(wc), fake, None, 8, ctypes.c_void_p(0x200000),
                            fake, 1 << 30, None)
    assert st == B.MOE_ERR_INVALID_ARG               # weights missing
    full = B.MoeWeightsC(*([fake] * 12))
    need = B.moe_workspace_size(cfg, 8)
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), fake, None, 8,
                              ctypes.c_void_p(0x200000), None, need, None) == B.MOE_ERR_WORKSPACE
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), fake, None, 8,
                              ctypes.c_void_p(0x200000), fake, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), fake, None, 8,
                              ctypes.c_void_p(0x200000), ctypes.c_void_p(0x100010), need, None) == B.MOE_ERR_WORKSPACE
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), fake, None, 8, fake, fake, need,
                              None) == B.MOE_ERR_INVALID_ARG   # y aliases x
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), fake, None, -1, fake, fake, need,
                              None) == B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op that succeeds without a workspace
    assert B._lib.moe_forward(ctypes.byref(cc), ctypes.byref(full), None, None, 0, None, None, 0,
                              None) == B.MOE_OK
    hc = B.config_c(C.SMALL_WORKLOADS["hash_small"].cfg)
    nohash = B.MoeWeightsC(*([fake] * 11 + [None]))
    assert B._lib.moe_forward(ctypes.byref(hc), ctypes.byref(nohash), fake, fake, 8,
                              ctypes.c_void_p(0x200000), fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG


def test_workspace_layout_is_aligned_and_disjoint():
    for wl in list(C.FULL_WORKLOADS.values()) + list(C.SMALL_WORKLOADS.values()):
        cfg, T = wl.cfg, wl.T
        lay = B.moe_workspace_layout(cfg, T)
        k, E = cfg.n_activated_experts, cfg.n_routed_experts
        rows = T * k + T * cfg.n_shared_experts
        es = 4 if cfg.act_dtype == "f32" else 2
        sizes = {"route_weights": 4 * T * k, "route_indices": 4 * T * k, "counts": 4 * E,
                 "offsets": 4 * (E + 1), "sorted_tok": 4 * (T * k + T), "sorted_slot": 4 * T * k,
                 "sorted_weight": 4 * T * k,
                 "inverse": 4 * T * k, "tiles": 16 * lay["max_tiles"], "tile_count": 4, "flags": 16,
                 "h": es * rows * cfg.moe_inter_dim, "yrows": es * rows * cfg.dim,
                 # at least one partial-logit plane for the split bf16 router
                 "route_logits": 4 * T * E if (cfg.route_mode == "learned"
                                               and cfg.act_dtype == "bf16") else 0,
                 "perm_hist": 4 * (-(-T * k // 256) + 1) * E}
        spans = sorted((lay[n], lay[n] + s) for n, s in sizes.items())
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(lay[n] % 256 == 0 for n in sizes)
        assert spans[-1][1] <= lay["total_bytes"] == B.moe_workspace_size(cfg, T)
        # enough tiles for any routing: sum_e ceil(c_e/BM) <= T*k/BM + min(E, T*k)
        bm = lay["tile_rows"]
        n_sh = -(-T // bm) if cfg.n_shared_experts else 0
        assert lay["max_tiles"] >= n_sh + T * k // bm + min(E, T * k)


def test_tid2eid_builder_matches_oracle_on_zipf_vocab():
    p = synth.zipf_probs(32768, 1.1)
    table, load, mx, mn = B.moe_build_tid2eid(p, 64, 4)
    otable, of, omx, omn = oracle.tid2eid_greedy(p, 64, 4)
    np.testing.assert_array_equal(table, otable)
    np.testing.assert_array_equal(load, of)
    assert (mx, mn) == (omx, omn)


@pytest.mark.parametrize("m,n,k,seed", [(1000, 16, 3, 0), (257, 7, 7, 1), (50, 64, 1, 2)])
def test_tid2eid_builder_matches_oracle_with_ties(m, n, k, seed):
    rng = np.random.default_rng(seed)
    p = rng.integers(1, 6, size=m).astype(np.float64)       # many equal frequencies
    p /= p.sum()
    table, load, mx, mn = B.moe_build_tid2eid(p, n, k)
    otable, of, omx, omn = oracle.tid2eid_greedy(p, n, k)
    np.testing.assert_array_equal(table, otable)
    np.testing.assert_array_equal(load, of)


def test_tid2eid_builder_rejects_bad_input():
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid(np.array([0.5, np.nan]), 4, 2)
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid(np.array([0.5, -0.1]), 4, 2)
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid(np.array([0.5, 0.5]), 2, 3)


def test_multistart_builder_matches_oracle():
    rng = np.random.default_rng(21)
    m, n, k = 3000, 32, 4
    p = rng.dirichlet(np.ones(m) * 0.5)
    orders = np.stack([rng.permutation(m) for _ in range(5)])
    table, load, mx, mn, best = B.moe_build_tid2eid_multistart(p, n, k, orders)
    ot, of, omx, omn, obest = oracle.tid2eid_multistart(p, n, k, orders)
    assert best == obest
    np.testing.assert_array_equal(table, ot)
    np.testing.assert_allclose(load, of, rtol=0, atol=0)
    assert (mx, mn) == (omx, omn)


def test_multistart_builder_rejects_bad_orders():
    p = np.full(4, 0.25)
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid_multistart(p, 2, 1, [[0, 1, 2, 2]])      # not a permutation
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid_multistart(p, 2, 1, [[0, 1, 2, 4]])      # out of range
    with pytest.raises(B.MoEError):
        B.moe_build_tid2eid_multistart(p, 2, 1, np.zeros((0, 4), dtype=np.int64))


def test_update_bias_and_ngram_checks_before_any_launch():
    fake = ctypes.c_void_p(0x100000)
    cc = B.config_c(V3)
    ub = B._lib.moe_update_bias
    assert ub(None, fake, 16, ctypes.c_float(0.001), fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(cc), None, 16, ctypes.c_float(0.001), fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(cc), fake, 16, ctypes.c_float(0.001), None, None, None) == B.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(cc), fake, 0, ctypes.c_float(0.001), fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert ub(ctypes.byref(cc), fake, 16, ctypes.c_float(float("nan")), fake, None,
              None) == B.MOE_ERR_INVALID_ARG
    ng = C.NGRAM_BF16.cfg
    assert B.moe_validate_config(ng) == B.MOE_OK
    assert B.moe_validate_config(replace(ng, vocab_size=0)) == B.MOE_ERR_INVALID_ARG
    assert B.moe_validate_config(replace(ng, vocab_size=1 << 31)) == B.MOE_ERR_INVALID_ARG
    # the 2-gram forward needs its pair table
    full = B.MoeWeightsC(*([fake] * 12))
    assert B._lib.moe_forward(ctypes.byref(B.config_c(ng)), ctypes.byref(full), fake, None, 8,
                              ctypes.c_void_p(0x200000), fake, 1 << 30, None) == B.MOE_ERR_INVALID_ARG


def test_probes_check_before_any_launch():
    fake = ctypes.c_void_p(0x100000)
    assert B._lib.moe_probe_read(None, 1 << 20, fake, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_read(fake, 8, fake, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_read(ctypes.c_void_p(0x100004), 1 << 20, fake, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_mfma(0, 0, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_mfma(10, 4, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_mfma(10, -1, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert B._lib.moe_probe_mfma(10, 0, None, None, None) == B.MOE_ERR_INVALID_ARG


def test_fp8_expert_config_valid():
    cfg = replace(C.V41_FLASH_FP4_MX.cfg, expert_dtype="fp8", weight_layout="tiled")
    assert B.moe_validate_config(cfg) == B.MOE_OK


def test_redequant_argument_checks():
    """Host-side checks of moe_redequant_fp8 (no launch happens)."""
    fake = ctypes.c_void_p(16)
    f = B._lib.moe_redequant_fp8
    assert f(fake, fake, -1, 128, 128, fake, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert f(fake, fake, 1, 0, 128, fake, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert f(fake, fake, 1, 192, 128, fake, fake, fake, None) == B.MOE_ERR_UNSUPPORTED
    assert f(fake, fake, 1, 128, 64, fake, fake, fake, None) == B.MOE_ERR_UNSUPPORTED
    assert f(None, fake, 1, 128, 128, fake, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert f(fake, fake, 1, 128, 128, fake, fake, None, None) == B.MOE_ERR_INVALID_ARG
    assert f(None, None, 0, 128, 128, None, None, None, None) == B.MOE_OK


def test_forward_ex_argument_checks():
    """Host-side checks of moe_forward_ex (no launch happens): the side
    stream may not be the main stream, and a given event array must be full."""
    cfg = C.V41_FLASH_FP4_MX.cfg
    cfg_c = B.config_c(cfg)
    w = B.MoeWeightsC()
    fake = ctypes.c_void_p(0x100000)
    f = B._lib.moe_forward_ex
    s = ctypes.c_void_p(0x2000)
    assert f(ctypes.byref(cfg_c), ctypes.byref(w), fake, None, 64, fake, fake, 1 << 30, None,
             s, s) == B.MOE_ERR_INVALID_ARG
    events = (ctypes.c_void_p * (len(B.MOE_STAGES) + 1))()
    assert f(ctypes.byref(cfg_c), ctypes.byref(w), fake, None, 64, fake, fake, 1 << 30, events,
             s, None) == B.MOE_ERR_INVALID_ARG
    # T == 0 is a no-op that returns before any stream is touched
    assert f(ctypes.byref(cfg_c), ctypes.byref(w), fake, None, 0, fake, fake, 0, None,
             s, ctypes.c_void_p(0x3000)) == B.MOE_OK


def test_forward_ex_side_stream_error_returns_status():
    """With a side stream on a host where the HIP runtime has no usable
    device, moe_forward_ex passes every host check and then reports
    MOE_ERR_HIP from the side-stream set-up (event creation needs a device)
    instead of crashing; nothing is launched.  Skipped where a device exists."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the no-device path cannot be reached")
    cfg = C.V41_FLASH_FP4_MX.cfg
    cfg_c = B.config_c(cfg)
    fake = ctypes.c_void_p(0x100000)
    w = B.MoeWeightsC(*([fake] * 12))
    T = 64
    need = B.moe_workspace_size(cfg, T)
    st = B._lib.moe_forward_ex(ctypes.byref(cfg_c), ctypes.byref(w), fake, None, T,
                               ctypes.c_void_p(0x200000), fake, need, None,
                               ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000))
    assert st == B.MOE_ERR_HIP
