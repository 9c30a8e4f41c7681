"""Thin Python binding of the C ABI in include/moe.h (argument marshalling only).

Every function has the name of the C entry point it calls.  Device buffers
are torch tensors (PyTorch provides the device memory and the stream); all
arithmetic happens in the HIP library.  There is no fallback: if the library
is not built, importing this module raises.
"""

import ctypes
import os

import numpy as np
import torch  # loaded first so the library binds to the same HIP runtime as torch

from dataclasses import replace

from .config import ACT_QUANT, DTYPE, LAYOUT, ROUTE, SCORE, MoEConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_FLAG_TOKEN_ID_RANGE = 1
MOE_FLAG_EXPERT_RANGE = 2
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED_SYMBOLS = (
    "moe_status_string", "moe_validate_config", "moe_build_tid2eid", "moe_workspace_layout",
    "moe_workspace_size", "moe_route", "moe_permute", "moe_forward", "moe_forward_profiled",
    "moe_pack_weights", "moe_build_tid2eid_multistart", "moe_update_bias", "moe_probe_read",
    "moe_probe_mfma", "moe_redequant_fp8", "moe_forward_ex", "moe_forward_noalloc",
)
MOE_STAGES = ("route", "permute", "gemm1", "gemm2", "combine")


class MoeConfigC(ctypes.Structure):
    _fields_ = [
        ("dim", ctypes.c_int32), ("n_routed_experts", ctypes.c_int32),
        ("n_activated_experts", ctypes.c_int32), ("n_expert_groups", ctypes.c_int32),
        ("n_limited_groups", ctypes.c_int32), ("moe_inter_dim", ctypes.c_int32),
        ("n_shared_experts", ctypes.c_int32), ("score_func", ctypes.c_int32),
        ("route_scale", ctypes.c_float), ("renormalize", ctypes.c_int32),
        ("swiglu_limit", ctypes.c_float), ("route_mode", ctypes.c_int32),
        ("vocab_size", ctypes.c_int64), ("act_dtype", ctypes.c_int32),
        ("expert_dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32),
        ("act_quant", ctypes.c_int32),
    ]


class MoeWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gate_w", "gate_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "tid2eid")]


class MoeWsLayoutC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "total_bytes", "route_weights", "route_indices", "counts", "offsets", "sorted_tok",
        "sorted_slot", "sorted_weight", "inverse", "tiles", "tile_count", "flags",
        "route_logits", "perm_hist", "xq", "xq_scales", "hq", "hq_scales", "h", "yrows")] + [
        ("max_tiles", ctypes.c_int32), ("tile_rows", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    cfgp, wp = ctypes.POINTER(MoeConfigC), ctypes.POINTER(MoeWeightsC)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_validate_config.argtypes = [cfgp]
    lib.moe_build_tid2eid.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
    lib.moe_workspace_layout.argtypes = [cfgp, i64, ctypes.POINTER(MoeWsLayoutC)]
    lib.moe_workspace_size.restype = ctypes.c_size_t
    lib.moe_workspace_size.argtypes = [cfgp, i64]
    lib.moe_route.argtypes = [cfgp, wp, vp, vp, i64, vp, vp, vp]
    lib.moe_permute.argtypes = [cfgp, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_forward.argtypes = [cfgp, wp, vp, vp, i64, vp, vp, ctypes.c_size_t, vp]
    lib.moe_pack_weights.argtypes = [cfgp, wp, wp, vp]
    lib.moe_build_tid2eid_multistart.argtypes = [vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.moe_update_bias.argtypes = [cfgp, vp, i64, ctypes.c_float, vp, vp, vp]
    lib.moe_probe_read.argtypes = [vp, i64, vp, vp]
    lib.moe_probe_mfma.argtypes = [i32, i32, vp, vp, vp]
    lib.moe_redequant_fp8.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp]
    lib.moe_forward_profiled.argtypes = [cfgp, wp, vp, vp, i64, vp, vp, ctypes.c_size_t,
                                         ctypes.POINTER(ctypes.c_void_p), vp]
    lib.moe_forward_ex.argtypes = [cfgp, wp, vp, vp, i64, vp, vp, ctypes.c_size_t,
                                   ctypes.POINTER(ctypes.c_void_p), vp, vp]
    lib.moe_forward_noalloc.argtypes = [cfgp, wp, vp, vp, i64, vp, vp]
    for f in ("moe_validate_config", "moe_build_tid2eid", "moe_workspace_layout", "moe_route",
              "moe_permute", "moe_forward", "moe_forward_profiled", "moe_forward_ex",
              "moe_forward_noalloc",
              "moe_pack_weights",
              "moe_build_tid2eid_multistart", "moe_update_bias", "moe_probe_read",
              "moe_probe_mfma"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


_lib = _load()


class MoEError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")


def _check(status, where):
    if status != MOE_OK:
        raise MoEError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return ctypes.c_void_p(t.data_ptr())
    if isinstance(t, np.ndarray):
        return t.ctypes.data_as(ctypes.c_void_p)
    raise TypeError(type(t))


def _stream(stream):
    if isinstance(stream, int):              # a raw hipStream_t (0 = default stream)
        return ctypes.c_void_p(stream)
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def config_c(cfg: MoEConfig) -> MoeConfigC:
    return MoeConfigC(
        cfg.dim, cfg.n_routed_experts, cfg.n_activated_experts, cfg.n_expert_groups,
        cfg.n_limited_groups, cfg.moe_inter_dim, cfg.n_shared_experts, SCORE[cfg.score_func],
        cfg.route_scale, cfg.renormalize, cfg.swiglu_limit, ROUTE[cfg.route_mode],
        cfg.vocab_size, DTYPE[cfg.act_dtype], DTYPE[cfg.expert_dtype], LAYOUT[cfg.weight_layout],
        ACT_QUANT[cfg.act_quant])


def weights_c(layer: dict) -> MoeWeightsC:
    return MoeWeightsC(*[_ptr(layer.get(n)) for n in (
        "gate_w", "gate_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "tid2eid")])


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(int(status)).decode()


def moe_validate_config(cfg: MoEConfig) -> int:
    return _lib.moe_validate_config(ctypes.byref(config_c(cfg)))


def moe_build_tid2eid(p, n: int, k: int):
    """Greedy table on the host.  Returns (tid2eid int32 [m,k], load [n], max_vio, min_vio)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    m = p.shape[0]
    table = np.empty((m, k), dtype=np.int32)
    load = np.empty(n, dtype=np.float64)
    mx, mn = ctypes.c_double(), ctypes.c_double()
    _check(_lib.moe_build_tid2eid(_ptr(p), m, n, k, _ptr(table), _ptr(load), ctypes.byref(mx),
                                  ctypes.byref(mn)), "moe_build_tid2eid")
    return table, load, mx.value, mn.value


def moe_build_tid2eid_multistart(p, n: int, k: int, orders):
    """Multi-start greedy on the host.  orders: int64 [S, m] token orders.
    Returns (tid2eid, load, max_vio, min_vio, best_start)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    orders = np.ascontiguousarray(orders, dtype=np.int64)
    m = p.shape[0]
    table = np.empty((m, k), dtype=np.int32)
    load = np.empty(n, dtype=np.float64)
    mx, mn, best = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _check(_lib.moe_build_tid2eid_multistart(_ptr(p), m, n, k, _ptr(orders), orders.shape[0],
                                             _ptr(table), _ptr(load), ctypes.byref(mx),
                                             ctypes.byref(mn), ctypes.byref(best)),
           "moe_build_tid2eid_multistart")
    return table, load, mx.value, mn.value, best.value


def moe_update_bias(cfg: MoEConfig, counts, T: int, gamma: float, bias, stats=None, stream=None):
    """Sign step of the selection bias (device tensors; bias updated in place;
    stats: float64 [4] device tensor or None)."""
    _check(_lib.moe_update_bias(ctypes.byref(config_c(cfg)), _ptr(counts), T, gamma, _ptr(bias),
                                _ptr(stats), _stream(stream)), "moe_update_bias")


def moe_probe_read(buf, out, stream=None):
    _check(_lib.moe_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                               _stream(stream)), "moe_probe_read")


def moe_probe_mfma(iters: int, out, shape=0, stream=None) -> float:
    """Launch the MFMA probe (shape 0: 16x16x32 bf16, 1: 32x32x16 bf16,
    2: scaled 16x16x128 E4M3 x E2M1, 3: the same E4M3 x E4M3); returns the
    flops the launch performs."""
    flops = ctypes.c_double()
    _check(_lib.moe_probe_mfma(iters, shape, _ptr(out), ctypes.byref(flops), _stream(stream)),
           "moe_probe_mfma")
    return flops.value


def moe_workspace_layout(cfg: MoEConfig, T: int) -> dict:
    lay = MoeWsLayoutC()
    _check(_lib.moe_workspace_layout(ctypes.byref(config_c(cfg)), T, ctypes.byref(lay)),
           "moe_workspace_layout")
    return {name: getattr(lay, name) for name, _ in MoeWsLayoutC._fields_}


def moe_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _lib.moe_workspace_size(ctypes.byref(config_c(cfg)), T)


def moe_route(cfg: MoEConfig, layer: dict, x, token_ids, T: int, weights, indices, stream=None):
    _check(_lib.moe_route(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(layer)), _ptr(x),
                          _ptr(token_ids), T, _ptr(weights), _ptr(indices), _stream(stream)),
           "moe_route")


def moe_permute(cfg: MoEConfig, indices, T: int, counts, offsets, sorted_tok, sorted_slot,
                inverse, flags=None, stream=None):
    _check(_lib.moe_permute(ctypes.byref(config_c(cfg)), _ptr(indices), T, _ptr(counts),
                            _ptr(offsets), _ptr(sorted_tok), _ptr(sorted_slot), _ptr(inverse),
                            _ptr(flags), _stream(stream)), "moe_permute")


PACKED_MEMBERS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                  "sh_gate", "sh_up", "sh_down")


def moe_pack_weights(cfg: MoEConfig, src: dict, dst: dict, stream=None):
    _check(_lib.moe_pack_weights(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(src)),
                                 ctypes.byref(weights_c(dst)), _stream(stream)),
           "moe_pack_weights")


def pack_layer(cfg: MoEConfig, layer: dict, stream=None):
    """(cfg with weight_layout "tiled", a copy of `layer` whose expert matrices
    are freshly allocated tiled copies written by moe_pack_weights)."""
    out = dict(layer)
    for n in PACKED_MEMBERS:
        if layer.get(n) is not None:
            out[n] = torch.empty_like(layer[n])
    moe_pack_weights(cfg, layer, out, stream)
    return replace(cfg, weight_layout="tiled"), out


def moe_redequant_fp8(codes, scales, n_mat: int, N: int, K: int, fp8, block_scales, lossy,
                      stream=None):
    """FP4 [n_mat, N, K/2] codes + [n_mat, N, K/32] scales -> E4M3 codes in the
    FP8 expert layout, [n_mat, N/128, K/128] block scales and lossy flags."""
    _check(_lib.moe_redequant_fp8(_ptr(codes), _ptr(scales), n_mat, N, K, _ptr(fp8),
                                  _ptr(block_scales), _ptr(lossy), _stream(stream)),
           "moe_redequant_fp8")


def redequant_layer(cfg: MoEConfig, layer: dict, stream=None):
    """(cfg with FP8 experts and tiled weights, a copy of the FP4 `layer` whose
    routed matrices are re-dequantised to FP8 by moe_redequant_fp8 and whose
    shared matrices are tiled by moe_pack_weights, total lossy block count)."""
    if cfg.expert_dtype != "fp4" or cfg.weight_layout != "rows":
        raise ValueError("redequant_layer takes an FP4 layer in the row layout")
    out = dict(layer)
    shared = {n: layer.get(n) for n in ("sh_gate", "sh_up", "sh_down")}
    if cfg.n_shared_experts:
        dst = {n: torch.empty_like(v) for n, v in shared.items()}
        moe_pack_weights(cfg, shared, dst, stream)
        out.update(dst)
    E, d, I = cfg.n_routed_experts, cfg.dim, cfg.moe_inter_dim
    dev = layer["w_gate"].device
    lossy_total = 0
    for n, sn, N, K in (("w_gate", "s_gate", I, d), ("w_up", "s_up", I, d),
                        ("w_down", "s_down", d, I)):
        codes = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        bsc = torch.empty((E, N // 128, K // 128), dtype=torch.uint8, device=dev)
        lossy = torch.empty_like(bsc)
        moe_redequant_fp8(layer[n], layer[sn], E, N, K, codes, bsc, lossy, stream)
        out[n], out[sn] = codes, bsc
        lossy_total += int(lossy.sum())
    return replace(cfg, expert_dtype="fp8", weight_layout="tiled"), out, lossy_total


def moe_forward(cfg: MoEConfig, layer: dict, x, token_ids, T: int, y, ws, stream=None,
                ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.moe_forward(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(layer)), _ptr(x),
                            _ptr(token_ids), T, _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_forward")


def moe_forward_profiled(cfg: MoEConfig, layer: dict, x, token_ids, T: int, y, ws, events,
                         stream=None):
    """events: len(MOE_STAGES) + 1 raw hipEvent_t handles (see HipEvents)."""
    arr = (ctypes.c_void_p * len(events))(*events)
    _check(_lib.moe_forward_profiled(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(layer)),
                                     _ptr(x), _ptr(token_ids), T, _ptr(y), _ptr(ws),
                                     ws.numel() * ws.element_size(), arr, _stream(stream)),
           "moe_forward_profiled")


def moe_forward_ex(cfg: MoEConfig, layer: dict, x, token_ids, T: int, y, ws, events=None,
                   stream=None, side_stream=None):
    """events: None or len(MOE_STAGES) + 1 raw hipEvent_t handles; side_stream:
    None, or a torch stream / raw handle other than `stream`."""
    arr = (ctypes.c_void_p * len(events))(*events) if events is not None else None
    side = None if side_stream is None else _stream(side_stream)
    _check(_lib.moe_forward_ex(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(layer)),
                               _ptr(x), _ptr(token_ids), T, _ptr(y), _ptr(ws),
                               ws.numel() * ws.element_size(), arr, _stream(stream), side),
           "moe_forward_ex")


def moe_forward_noalloc(cfg: MoEConfig, layer: dict, x, token_ids, T: int, y, stream=None):
    """moe_forward on the library's own device array (no workspace argument)."""
    _check(_lib.moe_forward_noalloc(ctypes.byref(config_c(cfg)), ctypes.byref(weights_c(layer)),
                                    _ptr(x), _ptr(token_ids), T, _ptr(y), _stream(stream)),
           "moe_forward_noalloc")


class HipEvents:
    """Raw HIP timing events from the HIP runtime torch already loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[a]),
                                        ctypes.c_void_p(self.handles[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.handles = []


# ---------------------------------------------------------------------------
# Convenience views of a forward workspace (no computation).

def alloc_workspace(cfg: MoEConfig, T: int, device="cuda"):
    size = moe_workspace_size(cfg, T)
    if size == 0:
        raise MoEError(moe_validate_config(cfg), "moe_workspace_size")
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(size, dtype=torch.uint8, device=device)


def workspace_views(cfg: MoEConfig, T: int, ws):
    """Typed views of the routing, permutation and intermediate buffers."""
    lay = moe_workspace_layout(cfg, T)
    k, E = cfg.n_activated_experts, cfg.n_routed_experts
    rows = T * k + T * cfg.n_shared_experts
    edt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16

    def view(off, n, dtype):
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype)

    out = {
        "route_weights": view(lay["route_weights"], T * k, torch.float32).view(T, k),
        "route_indices": view(lay["route_indices"], T * k, torch.int32).view(T, k),
        "counts": view(lay["counts"], E, torch.int32),
        "offsets": view(lay["offsets"], E + 1, torch.int32),
        "sorted_tok": view(lay["sorted_tok"], T * k + T, torch.int32),
        "sorted_slot": view(lay["sorted_slot"], T * k, torch.int32),
        "sorted_weight": view(lay["sorted_weight"], T * k, torch.float32),
        "inverse": view(lay["inverse"], T * k, torch.int32).view(T, k),
        "tiles": view(lay["tiles"], 4 * lay["max_tiles"], torch.int32).view(-1, 4),
        "tile_count": view(lay["tile_count"], 1, torch.int32),
        "flags": view(lay["flags"], 4, torch.int32),
        "perm_hist": view(lay["perm_hist"], (-(-T * k // 256) + 1) * E, torch.int32),
        "h": view(lay["h"], rows * cfg.moe_inter_dim, edt).view(rows, cfg.moe_inter_dim),
        "yrows": view(lay["yrows"], rows * cfg.dim, edt).view(rows, cfg.dim),
        "layout": lay,
    }
    if cfg.act_quant == "mxfp8":
        I = cfg.moe_inter_dim
        out["xq"] = view(lay["xq"], T * cfg.dim, torch.uint8).view(T, cfg.dim)
        out["xq_scales"] = view(lay["xq_scales"], T * cfg.dim // 32, torch.uint8).view(T, -1)
        out["hq"] = view(lay["hq"], T * k * I, torch.uint8).view(T * k, I)
        out["hq_scales"] = view(lay["hq_scales"], T * k * I // 32, torch.uint8).view(T * k, -1)
    return out
