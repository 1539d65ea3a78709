"""ctypes binding of libmoe_route.so: argument marshalling only.

Every function named ``moe_*`` here calls the C entry point of the same name
declared in include/moe_route.h; all work runs in the library's HIP kernels.
PyTorch supplies device memory (tensors are passed by ``data_ptr()``) and the
current stream.  A missing library is an ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch  # loaded first so the library binds to the same HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_route.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MODES = {"standard": 0, "lore": 1, "stall_free": 2, "floe": 3}
MOE_UP_DENSE, MOE_UP_INT2_G64 = 0, 1
LAYOUTS = {"rows": 0, "mfma16": 1}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode()} (status {status})")


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("lore_rank", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("shared_gate", ctypes.c_int32), ("floe_keep", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("up_format", ctypes.c_int),
                ("tie_margin", ctypes.c_float), ("weight_layout", ctypes.c_int)]


_WEIGHT_FIELDS = ["w_router", "w_gate", "w_up", "w_down", "up_q", "up_scale", "up_zero",
                  "ws_gate", "ws_up", "ws_down", "w_shared_gate", "lore_A", "lore_B"]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


_DEBUG_FIELDS = ["topk_ids", "topk_w", "exact", "flags", "logits", "mass", "expert_offsets",
                 "perm", "floe_keep"]


KERNELS = {"none": 0, "route": 1, "permute": 2, "expert_gate_up": 3, "expert_down": 4,
           "floe_up": 5, "floe_select": 6, "floe_gate": 7, "floe_down": 8, "combine": 9,
           "shared_ffn": 10}


class MoeDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _DEBUG_FIELDS] + [
        ("prof_start", ctypes.c_void_p), ("prof_stop", ctypes.c_void_p),
        ("prof_kernel", ctypes.c_int32)]


class MoeOffloadCost(ctypes.Structure):
    _fields_ = [("pcie_bytes_per_s", ctypes.c_double), ("gpu_expert_s", ctypes.c_double),
                ("cpu_expert_s", ctypes.c_double), ("cpu_pair_s", ctypes.c_double),
                ("cpu_threads", ctypes.c_int32), ("queue_aware", ctypes.c_int32)]


class MoeOffloadStats(ctypes.Structure):
    _fields_ = [("missed_experts", ctypes.c_int32), ("fetched_experts", ctypes.c_int32),
                ("host_experts", ctypes.c_int32), ("host_pairs", ctypes.c_int32),
                ("route_ms", ctypes.c_double), ("host_ms", ctypes.c_double),
                ("parallel_ms", ctypes.c_double), ("wall_ms", ctypes.c_double),
                ("decision", ctypes.c_void_p), ("gpu_start", ctypes.c_void_p),
                ("gpu_stop", ctypes.c_void_p)]


OFFLOAD_NONE, OFFLOAD_FETCH, OFFLOAD_HOST = 0, 1, 2


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run sparse_moe_layer_route_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D, Wp, Dbg = ctypes.POINTER(MoeDims), ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeDebug)
    sig = {
        "moe_abi_version": ([], ctypes.c_int),
        "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "moe_workspace_size": ([D, I32, ctypes.c_int, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_route": ([D, I32, P, P, P, I64, ctypes.c_int, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_prefetch_mask": ([D, I32, P, P, P, P, P, P], ctypes.c_int),
        "moe_pack_size": ([I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_pack_weights": ([I32, I32, I32, P, P, P], ctypes.c_int),
        "moe_prefetch_adaptive": ([D, I32, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P],
                                  ctypes.c_int),
        "moe_permute": ([I32, I32, I32, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_expert_ffn": ([D, I32, P, Wp, ctypes.c_int, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_lore_surrogate": ([D, I32, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_floe_predict": ([D, I32, P, Wp, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_floe_pack": ([D, I32, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_lore_targets": ([D, I32, P, Wp, I32, P, P, SZ, P], ctypes.c_int),
        "moe_lore_fit_size": ([I32, I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_lore_fit": ([D, I32, P, P, I32, I32, I32, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_combine": ([D, I32, P, P, P, P, P, P, P, P, P], ctypes.c_int),
        "moe_layer_forward": ([D, I32, P, Wp, P, I64, ctypes.c_int, P, Dbg, P, SZ, P], ctypes.c_int),
        "moe_layer_forward_noalloc": ([D, I32, P, Wp, P, I64, ctypes.c_int, P, P], ctypes.c_int),
        "moe_offload_plan": ([D, P, P, ctypes.POINTER(MoeOffloadCost), P], ctypes.c_int),
        "moe_offload_workspace_size": ([D, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
                                       ctypes.c_int),
        "moe_host_ffn_workspace_size": ([D, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_host_expert_ffn": ([D, I32, P, Wp, I32, P, P, I32, P, P, SZ], ctypes.c_int),
        "moe_layer_forward_offload": ([D, I32, P, Wp, Wp, P, ctypes.POINTER(MoeOffloadCost), P, P,
                                       SZ, P, SZ, ctypes.POINTER(MoeOffloadStats), P],
                                      ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()
EXPORTED = ("moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_route",
            "moe_prefetch_mask", "moe_prefetch_adaptive", "moe_pack_size", "moe_pack_weights",
            "moe_permute", "moe_floe_predict", "moe_floe_pack", "moe_lore_targets",
            "moe_lore_fit_size", "moe_lore_fit", "moe_expert_ffn", "moe_lore_surrogate",
            "moe_combine", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_offload_plan",
            "moe_offload_workspace_size", "moe_host_ffn_workspace_size", "moe_host_expert_ffn",
            "moe_layer_forward_offload")


# ------------------------------------------------------------------ helpers --
@dataclasses.dataclass
class Dims:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int = 0
    shared_inter: int = 0
    lore_rank: int = 0
    renormalize: bool = False
    shared_gate: bool = False
    floe_keep: int = 0
    dtype: str = "bf16"
    up_format: str = "dense"
    tie_margin: float = 1e-4
    weight_layout: str = "rows"      # "rows" or "mfma16" (see pack_weights)

    def c(self) -> MoeDims:
        return MoeDims(self.hidden, self.n_experts, self.top_k, self.inter, self.n_shared,
                       self.shared_inter, self.lore_rank, int(self.renormalize),
                       int(self.shared_gate), self.floe_keep,
                       MOE_BF16 if self.dtype == "bf16" else MOE_F32,
                       MOE_UP_INT2_G64 if self.up_format == "int2_g64" else MOE_UP_DENSE,
                       self.tie_margin, LAYOUTS[self.weight_layout])


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _dims(d) -> MoeDims:
    return d.c() if isinstance(d, Dims) else d


# ------------------------------------------------------------- entry points --
def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_workspace_size(dims, T: int, mode) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_workspace_size(ctypes.byref(_dims(dims)), T, _mode(mode), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def moe_route(dims, T, x, w_router, resident, resident_stride, mode, topk_ids, topk_w, exact,
              flags, logits, mass=None, stream=None):
    _check(_lib.moe_route(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(w_router), _ptr(resident),
                          resident_stride, _mode(mode), _ptr(topk_ids), _ptr(topk_w), _ptr(exact),
                          _ptr(flags), _ptr(logits), _ptr(mass), _stream(stream)), "moe_route")


def moe_prefetch_mask(dims, T, x, w_prefetch, delta, mask_out, flags, stream=None):
    _check(_lib.moe_prefetch_mask(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(w_prefetch),
                                  _ptr(delta), _ptr(mask_out), _ptr(flags), _stream(stream)),
           "moe_prefetch_mask")


def moe_prefetch_adaptive(dims, T, x, w_prefetch, w_delta, theta, tau, delta_out, mask_out, flags,
                          topk_ids=None, delta_star=None, overlap=None, stream=None):
    _check(_lib.moe_prefetch_adaptive(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(w_prefetch),
                                      _ptr(w_delta), _ptr(theta), float(tau), _ptr(topk_ids),
                                      _ptr(delta_out), _ptr(mask_out), _ptr(flags),
                                      _ptr(delta_star), _ptr(overlap), _stream(stream)),
           "moe_prefetch_adaptive")


def moe_pack_size(groups, rows, cols) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_pack_size(groups, rows, cols, ctypes.byref(n)), "moe_pack_size")
    return n.value


def moe_pack_weights(groups, rows, cols, src, dst, stream=None):
    _check(_lib.moe_pack_weights(groups, rows, cols, _ptr(src), _ptr(dst), _stream(stream)),
           "moe_pack_weights")


# (groups, rows, cols) of each expert matrix that MOE_LAYOUT_MFMA16 packs
def _packed_shapes(d: "Dims"):
    E, H, I, ns, Is = d.n_experts, d.hidden, d.inter, d.n_shared, d.shared_inter
    shapes = {"w_gate": (E, I, H), "w_up": (E, I, H), "w_down": (E, H, I)}
    if ns > 0:
        shapes.update(ws_gate=(ns, Is, H), ws_up=(ns, Is, H), ws_down=(ns, H, Is))
    return shapes


def pack_weights(dims: "Dims", w: Dict[str, torch.Tensor], stream=None) -> Dict[str, torch.Tensor]:
    """A copy of the weight dict with the routed and shared expert matrices
    packed fragment-major (moe_pack_weights); use it with
    dataclasses.replace(dims, weight_layout="mfma16")."""
    if dims.dtype != "bf16":
        raise ValueError("the fragment-major layout holds bf16 weights only")
    out = dict(w)
    for name, (g, r, c) in _packed_shapes(dims).items():
        src = w[name]
        if src.element_size() != 2:
            raise ValueError(f"{name}: expected 2-byte (bf16) elements")
        if src.numel() != g * r * c:
            raise ValueError(f"{name}: expected {g}x{r}x{c} elements, got {src.numel()}")
        dst = torch.empty(moe_pack_size(g, r, c) // 2, dtype=src.dtype, device=src.device)
        moe_pack_weights(g, r, c, src, dst, stream)
        out[name] = dst
    return out


def moe_floe_predict(dims, T, h_prev, w, topk_ids, keep_out, flags, ws, stream=None):
    ws_ = weights_struct(w) if isinstance(w, dict) else w
    _check(_lib.moe_floe_predict(ctypes.byref(_dims(dims)), T, _ptr(h_prev), ctypes.byref(ws_),
                                 _ptr(topk_ids), _ptr(keep_out), _ptr(flags), _ptr(ws), ws.numel(),
                                 _stream(stream)), "moe_floe_predict")


def moe_floe_pack(dims, T, topk_ids, keep, w_gate, w_down, gate_out, down_out, stream=None):
    _check(_lib.moe_floe_pack(ctypes.byref(_dims(dims)), T, _ptr(topk_ids), _ptr(keep), _ptr(w_gate),
                              _ptr(w_down), _ptr(gate_out), _ptr(down_out), _stream(stream)),
           "moe_floe_pack")


def moe_lore_targets(dims, N, h_cal, w, expert, resid_out, ws, stream=None):
    ws_ = weights_struct(w) if isinstance(w, dict) else w
    _check(_lib.moe_lore_targets(ctypes.byref(_dims(dims)), N, _ptr(h_cal), ctypes.byref(ws_), expert,
                                 _ptr(resid_out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_lore_targets")


def moe_lore_fit_size(hidden, N, rank, cols) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_lore_fit_size(hidden, N, rank, cols, ctypes.byref(n)), "moe_lore_fit_size")
    return n.value


def moe_lore_fit(dims, N, h_cal, resid, rank, cols, n_iter, omega, lore_A_out, lore_B_out,
                 sigma_out, err_out, ws, stream=None):
    _check(_lib.moe_lore_fit(ctypes.byref(_dims(dims)), N, _ptr(h_cal), _ptr(resid), rank, cols,
                             n_iter, _ptr(omega), _ptr(lore_A_out), _ptr(lore_B_out),
                             _ptr(sigma_out), _ptr(err_out), _ptr(ws), ws.numel(),
                             _stream(stream)), "moe_lore_fit")


def moe_permute(T, k, E, topk_ids, exact, expert_offsets, perm, inv, ws=None, stream=None):
    _check(_lib.moe_permute(T, k, E, _ptr(topk_ids), _ptr(exact), _ptr(expert_offsets), _ptr(perm),
                            _ptr(inv), _ptr(ws), ws.numel() if ws is not None else 0,
                            _stream(stream)), "moe_permute")


def weights_struct(w: Dict[str, torch.Tensor]) -> MoeWeights:
    return MoeWeights(*[_ptr(w.get(n)) for n in _WEIGHT_FIELDS])


def moe_expert_ffn(dims, T, x, weights, mode, expert_offsets, perm, y_perm, y_shared, shared_gate,
                   ws, floe_keep=None, flags=None, stream=None):
    ws_struct = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    _check(_lib.moe_expert_ffn(ctypes.byref(_dims(dims)), T, _ptr(x), ctypes.byref(ws_struct),
                               _mode(mode), _ptr(expert_offsets), _ptr(perm), _ptr(y_perm),
                               _ptr(y_shared), _ptr(shared_gate), _ptr(floe_keep), _ptr(flags),
                               _ptr(ws), ws.numel(), _stream(stream)), "moe_expert_ffn")


def moe_lore_surrogate(dims, T, x, topk_ids, exact, lore_A, lore_B, lore_out, stream=None):
    _check(_lib.moe_lore_surrogate(ctypes.byref(_dims(dims)), T, _ptr(x), _ptr(topk_ids),
                                   _ptr(exact), _ptr(lore_A), _ptr(lore_B), _ptr(lore_out),
                                   _stream(stream)), "moe_lore_surrogate")


def moe_combine(dims, T, y_perm, inv, topk_w, exact, y_shared, shared_gate, lore_out, out,
                stream=None):
    _check(_lib.moe_combine(ctypes.byref(_dims(dims)), T, _ptr(y_perm), _ptr(inv), _ptr(topk_w),
                            _ptr(exact), _ptr(y_shared), _ptr(shared_gate), _ptr(lore_out),
                            _ptr(out), _stream(stream)), "moe_combine")


def moe_layer_forward(dims, T, x, weights, resident, resident_stride, mode, out, ws, debug=None,
                      stream=None):
    ws_struct = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    dbg = None
    if isinstance(debug, MoeDebug):
        dbg = ctypes.byref(debug)
    elif debug is not None:
        prof = debug.get("prof")        # (start_event, stop_event, kernel name): raw hipEvent_t
        dbg = ctypes.byref(MoeDebug(*[_ptr(debug.get(n)) for n in _DEBUG_FIELDS],
                                    prof[0] if prof else None, prof[1] if prof else None,
                                    KERNELS[prof[2]] if prof else 0))
    _check(_lib.moe_layer_forward(ctypes.byref(_dims(dims)), T, _ptr(x), ctypes.byref(ws_struct),
                                  _ptr(resident), resident_stride, _mode(mode), _ptr(out), dbg,
                                  _ptr(ws), ws.numel(), _stream(stream)), "moe_layer_forward")


NOALLOC_SCRATCH_BYTES = 128 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def moe_layer_forward_noalloc(dims, T, x, weights, resident, resident_stride, mode, out,
                              stream=None):
    ws_struct = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(_dims(dims)), T, _ptr(x),
                                          ctypes.byref(ws_struct), _ptr(resident), resident_stride,
                                          _mode(mode), _ptr(out), _stream(stream)),
           "moe_layer_forward_noalloc")


# ------------------------------------------------- exact miss execution --
def _hptr(t):
    """Address of a host buffer: a contiguous CPU tensor or numpy array."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if t.is_cuda:
            raise ValueError("tensor must live in host memory")
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return t.data_ptr()
    import numpy as np
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return t.ctypes.data
    raise TypeError("expected a CPU torch.Tensor or a numpy array")


def offload_cost(pcie_bytes_per_s, gpu_expert_s, cpu_pair_s, cpu_threads=0,
                 cpu_expert_s=0.0, queue_aware=False) -> MoeOffloadCost:
    return MoeOffloadCost(float(pcie_bytes_per_s), float(gpu_expert_s), float(cpu_expert_s),
                          float(cpu_pair_s), int(cpu_threads), int(bool(queue_aware)))


def moe_offload_plan(dims, tokens, resident: int, cost: MoeOffloadCost):
    """Cost-rule decision per expert (OFFLOAD_NONE / FETCH / HOST), host only."""
    import numpy as np
    d = _dims(dims)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    if tok.shape != (d.n_experts,):
        raise ValueError("tokens must hold one count per expert")
    res = (ctypes.c_uint64 * 1)(int(resident) & (2**64 - 1))
    dec = np.zeros(d.n_experts, dtype=np.uint8)
    _check(_lib.moe_offload_plan(ctypes.byref(d), tok.ctypes.data, ctypes.addressof(res),
                                 ctypes.byref(cost), dec.ctypes.data), "moe_offload_plan")
    return dec


def moe_offload_workspace_size(dims, T: int):
    dev, host = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.moe_offload_workspace_size(ctypes.byref(_dims(dims)), T, ctypes.byref(dev),
                                           ctypes.byref(host)), "moe_offload_workspace_size")
    return dev.value, host.value


def moe_host_ffn_workspace_size(dims, n: int) -> int:
    b = ctypes.c_size_t(0)
    _check(_lib.moe_host_ffn_workspace_size(ctypes.byref(_dims(dims)), n, ctypes.byref(b)),
           "moe_host_ffn_workspace_size")
    return b.value


def _host_weights(w) -> MoeWeights:
    if isinstance(w, MoeWeights):
        return w
    st = MoeWeights()
    for n in ("w_gate", "w_up", "w_down"):
        setattr(st, n, _hptr(w[n]))
    return st


def moe_host_expert_ffn(dims, T, x, host_weights, tok, expert, threads, y_out, host_ws):
    """Host SwiGLU FFN of (token, expert) pairs; every buffer in host memory."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tok, dtype=np.int32))
    e = np.ascontiguousarray(np.asarray(expert, dtype=np.int32))
    if t.shape != e.shape or t.ndim != 1:
        raise ValueError("tok and expert must be 1-D of the same length")
    hw = _host_weights(host_weights)
    nbytes = host_ws.numel() * host_ws.element_size() if isinstance(host_ws, torch.Tensor) \
        else host_ws.nbytes
    _check(_lib.moe_host_expert_ffn(ctypes.byref(_dims(dims)), T, _hptr(x), ctypes.byref(hw),
                                    len(t), t.ctypes.data, e.ctypes.data, int(threads),
                                    _hptr(y_out), _hptr(host_ws), nbytes),
           "moe_host_expert_ffn")


def moe_layer_forward_offload(dims, T, x, weights, host_weights, resident: int,
                              cost: MoeOffloadCost, out, ws, host_ws, stats=None, stream=None):
    """Layer forward with missed experts fetched or run on the host (exact).

    weights: device tensors (the expert slots are written for fetched
    experts); host_weights: pinned CPU tensors w_gate / w_up / w_down;
    host_ws: pinned CPU uint8 tensor; stats: a MoeOffloadStats or None."""
    ws_struct = weights if isinstance(weights, MoeWeights) else weights_struct(weights)
    hw = _host_weights(host_weights)
    res = (ctypes.c_uint64 * 1)(int(resident) & (2**64 - 1))
    _check(_lib.moe_layer_forward_offload(
        ctypes.byref(_dims(dims)), T, _ptr(x), ctypes.byref(ws_struct), ctypes.byref(hw),
        ctypes.addressof(res), ctypes.byref(cost), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _hptr(host_ws), host_ws.numel() * host_ws.element_size(),
        ctypes.byref(stats) if stats is not None else None, _stream(stream)),
        "moe_layer_forward_offload")
