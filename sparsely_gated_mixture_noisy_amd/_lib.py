"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  Tensors are torch tensors on the current HIP device; outputs are
allocated here with torch and filled by the library on torch's current stream.
The library must be built (python -m sparsely_gated_mixture_noisy_amd.build);
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional

import torch

from .inputs import MoEConfig

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_F32, MOE_BF16 = 0, 1
MOE_FFN_RELU, MOE_FFN_SWIGLU = 0, 1


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed with status {status}: {detail}")
        self.status = status


class moe_config(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("d_hidden", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("k_groups", ctypes.c_int32), ("k_per_group", ctypes.c_int32),
                ("noisy", ctypes.c_int32), ("ffn", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


class moe_params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_gate", "w_noise", "bias", "w_gate_p", "w_noise_p", "w1", "w3", "w2",
                 "w_packed", "w_gate_packed")]


class moe_noise(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_void_p), ("eps_p", ctypes.c_void_p),
                ("seed", ctypes.c_uint64), ("in_kernel", ctypes.c_int32)]


class moe_outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("y", "topk_idx", "topk_gate", "counts", "importance", "load", "balance",
                 "thr", "offsets", "perm", "inv", "y_sorted")]


class moe_mask_outputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("y", "counts", "offsets", "perm", "tok_offsets", "slot_expert", "slot_gate",
                 "slot_row", "importance", "load", "balance")]


class moe_saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_gate", "thr", "offsets", "perm", "inv", "y_sorted",
                 "importance", "load")]


class moe_grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_gate", "dw_noise", "dbias", "dw1", "dw3", "dw2", "dw_gate_p",
                 "dw_noise_p")]


_P = ctypes.c_void_p
_SIGS = {
    "moe_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(moe_config)]),
    "moe_gate": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, ctypes.POINTER(moe_params),
                                ctypes.POINTER(moe_noise), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, _P, _P,
                                      ctypes.POINTER(moe_params), _P, _P, ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, _P, _P, _P, _P]),
    "moe_balance_loss": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, ctypes.POINTER(moe_params),
                                        _P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P,
                                        _P, _P, ctypes.c_size_t, _P]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, ctypes.POINTER(moe_params),
                                   ctypes.POINTER(moe_noise), ctypes.c_float, ctypes.c_float,
                                   ctypes.POINTER(moe_outputs), _P, ctypes.c_size_t, _P]),
    "moe_forward_static": (ctypes.c_int, [ctypes.POINTER(moe_config), _P,
                                          ctypes.POINTER(moe_params), ctypes.POINTER(moe_noise),
                                          ctypes.c_float, ctypes.c_float,
                                          ctypes.POINTER(moe_outputs), _P]),
    "moe_mask_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(moe_config), ctypes.c_int32]),
    "moe_forward_mask": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, ctypes.POINTER(moe_params),
                                        ctypes.POINTER(moe_noise), ctypes.c_int32, _P,
                                        ctypes.c_float, ctypes.c_float,
                                        ctypes.POINTER(moe_mask_outputs), _P, ctypes.c_size_t, _P]),
    "moe_packed_experts_size": (ctypes.c_size_t, [ctypes.POINTER(moe_config)]),
    "moe_pack_experts": (ctypes.c_int, [ctypes.POINTER(moe_config), ctypes.POINTER(moe_params),
                                        _P, _P]),
    "moe_packed_gate_size": (ctypes.c_size_t, [ctypes.POINTER(moe_config)]),
    "moe_pack_gate": (ctypes.c_int, [ctypes.POINTER(moe_config), ctypes.POINTER(moe_params),
                                     _P, _P]),
    "moe_backward_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(moe_config)]),
    "moe_backward": (ctypes.c_int, [ctypes.POINTER(moe_config), _P, ctypes.POINTER(moe_params),
                                    ctypes.POINTER(moe_noise), ctypes.POINTER(moe_saved), _P,
                                    ctypes.c_float, ctypes.c_float, ctypes.POINTER(moe_grads), _P,
                                    ctypes.c_size_t, _P]),
    "moe_draw_noise": (ctypes.c_int, [ctypes.POINTER(moe_config), ctypes.c_uint64, _P, _P, _P]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libmoe.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparsely_gated_mixture_noisy_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def _check(status: int, what: str):
    if status != MOE_OK:
        lib = load()
        raise MoEError(status, what, lib.moe_last_error().decode())


def make_config(cfg: MoEConfig, tokens: Optional[int] = None) -> moe_config:
    return moe_config(
        tokens=cfg.tokens if tokens is None else tokens, d_model=cfg.d_model,
        n_experts=cfg.n_experts, d_hidden=cfg.d_hidden, top_k=cfg.top_k,
        n_groups=cfg.n_groups, k_groups=cfg.k_groups, k_per_group=cfg.k_per_group,
        noisy=1 if cfg.noisy else 0,
        ffn=MOE_FFN_SWIGLU if cfg.ffn == "swiglu" else MOE_FFN_RELU,
        dtype=MOE_BF16 if cfg.dtype == "bf16" else MOE_F32, capacity=cfg.capacity)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_params(p: Dict[str, Optional[torch.Tensor]]) -> moe_params:
    return moe_params(**{n: _ptr(p.get(n)) for n, _ in moe_params._fields_})


def make_noise(p: Dict[str, Optional[torch.Tensor]]) -> moe_noise:
    """The noise tensors of p, or, when p holds "noise_seed", noise drawn
    inside the kernels from that seed (the tensors are then not read)."""
    seed = p.get("noise_seed")
    if seed is not None:
        return moe_noise(eps=None, eps_p=None, seed=int(seed), in_kernel=1)
    return moe_noise(eps=_ptr(p.get("eps")), eps_p=_ptr(p.get("eps_p")), seed=0, in_kernel=0)


def draw_noise(cfg: MoEConfig, seed: int, tokens: Optional[int] = None, device="cuda"):
    """The generator's draws for `seed` as tensors: (eps, eps_p)."""
    T = cfg.tokens if tokens is None else tokens
    if cfg.hierarchical:
        eps = torch.empty((T, cfg.n_groups, cfg.experts_per_group), dtype=torch.float32,
                          device=device)
        eps_p = torch.empty((T, cfg.n_groups), dtype=torch.float32, device=device)
    else:
        eps = torch.empty((T, cfg.n_experts), dtype=torch.float32, device=device)
        eps_p = None
    c = make_config(cfg, T)
    _check(load().moe_draw_noise(ctypes.byref(c), int(seed), _ptr(eps), _ptr(eps_p), _stream()),
           "moe_draw_noise")
    return eps, eps_p


def packed_experts_size(cfg: MoEConfig) -> int:
    c = make_config(cfg)
    return int(load().moe_packed_experts_size(ctypes.byref(c)))


def pack_experts(cfg: MoEConfig, params) -> Optional[torch.Tensor]:
    """The expert tables w1/w2 repacked for the expert kernel's weight
    stream (a bf16 tensor on the tables' device), or None when the layer has
    no packed form."""
    n = packed_experts_size(cfg)
    if n == 0:
        return None
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=params["w1"].device)
    c, p = make_config(cfg), make_params(params)
    _check(load().moe_pack_experts(ctypes.byref(c), ctypes.byref(p), _ptr(out), _stream()),
           "moe_pack_experts")
    return out


def packed_gate_size(cfg: MoEConfig) -> int:
    c = make_config(cfg)
    return int(load().moe_packed_gate_size(ctypes.byref(c)))


def pack_gate(cfg: MoEConfig, params) -> Optional[torch.Tensor]:
    """The gate tables w_gate/w_noise repacked for the gate kernels' table
    stream (a bf16 tensor on the tables' device), or None when the layer has
    no packed form."""
    n = packed_gate_size(cfg)
    if n == 0:
        return None
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=params["w_gate"].device)
    c, p = make_config(cfg), make_params(params)
    _check(load().moe_pack_gate(ctypes.byref(c), ctypes.byref(p), _ptr(out), _stream()),
           "moe_pack_gate")
    return out


def packed_params(cfg: MoEConfig, params):
    """params plus the packed expert and gate tables when the layer has them
    (w_packed, w_gate_packed): the form moe_forward reads them in at full
    speed.  The plain tables stay in the dict for the entry points that read
    them (the backward pass)."""
    out = dict(params)
    packed = pack_experts(cfg, params)
    if packed is not None:
        out["w_packed"] = packed
    gpacked = pack_gate(cfg, params)
    if gpacked is not None:
        out["w_gate_packed"] = gpacked
    return out


def workspace_size(cfg: MoEConfig, tokens: Optional[int] = None) -> int:
    c = make_config(cfg, tokens)
    return int(load().moe_workspace_size(ctypes.byref(c)))


class Workspace:
    """A 256-byte aligned device buffer of at least `nbytes` bytes."""

    def __init__(self, nbytes: int, device="cuda"):
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.ptr = (base + 255) & ~255
        self.nbytes = nbytes


def workspace(cfg: MoEConfig, tokens: Optional[int] = None, device="cuda") -> Workspace:
    return Workspace(workspace_size(cfg, tokens), device)


def _act_dtype(cfg: MoEConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def gate(cfg: MoEConfig, x, params, noise, ws: Optional[Workspace] = None, want_thr=True):
    T = x.shape[0]
    dev = x.device
    ws = ws or workspace(cfg, T, dev)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    g = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    thr = (torch.empty((T, 2), dtype=torch.float32, device=dev)
           if want_thr and not cfg.hierarchical else None)
    c, p, n = make_config(cfg, T), make_params(params), make_noise(noise)
    _check(load().moe_gate(ctypes.byref(c), _ptr(x), ctypes.byref(p), ctypes.byref(n), _ptr(idx),
                           _ptr(g), _ptr(thr), ws.ptr, ws.nbytes, _stream()), "moe_gate")
    return idx, g, thr


def route(cfg: MoEConfig, idx, x=None, ws: Optional[Workspace] = None):
    T = idx.shape[0]
    dev = idx.device
    ws = ws or workspace(cfg, T, dev)
    A = T * cfg.top_k
    counts = torch.empty(cfg.n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(A, dtype=torch.int32, device=dev)
    inv = torch.empty(A, dtype=torch.int32, device=dev)
    xs = (torch.empty((A, cfg.d_model), dtype=x.dtype, device=dev) if x is not None else None)
    c = make_config(cfg, T)
    _check(load().moe_route(ctypes.byref(c), _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                            _ptr(inv), _ptr(x), _ptr(xs), ws.ptr, ws.nbytes, _stream()),
           "moe_route")
    return counts, offsets, perm, inv, xs


def expert_ffn(cfg: MoEConfig, x, perm, offsets, params, tokens: Optional[int] = None,
               ws: Optional[Workspace] = None):
    """perm given: rows are x[perm[p] // k]; perm None: x is x_sorted [A][d]."""
    T = x.shape[0] if perm is not None else (tokens if tokens is not None else x.shape[0] // cfg.top_k)
    dev = x.device
    ws = ws or workspace(cfg, T, dev)
    ys = torch.empty((T * cfg.top_k, cfg.d_model), dtype=_act_dtype(cfg), device=dev)
    c, p = make_config(cfg, T), make_params(params)
    _check(load().moe_expert_ffn(ctypes.byref(c), _ptr(x), _ptr(perm), _ptr(offsets),
                                 ctypes.byref(p), _ptr(ys), ws.ptr, ws.nbytes, _stream()),
           "moe_expert_ffn")
    return ys


def combine(cfg: MoEConfig, y_sorted, inv, gates):
    T = gates.shape[0]
    y = torch.empty((T, cfg.d_model), dtype=_act_dtype(cfg), device=gates.device)
    c = make_config(cfg, T)
    _check(load().moe_combine(ctypes.byref(c), _ptr(y_sorted), _ptr(inv), _ptr(gates), _ptr(y),
                              _stream()), "moe_combine")
    return y


def balance_loss(cfg: MoEConfig, x, params, idx, gates, thr, perm, offsets, w_importance=1.0,
                 w_load=1.0, ws: Optional[Workspace] = None):
    T = gates.shape[0]
    dev = gates.device
    ws = ws or workspace(cfg, T, dev)
    imp = torch.empty(cfg.n_experts, dtype=torch.float32, device=dev)
    load_ = torch.empty(cfg.n_experts, dtype=torch.float32, device=dev)
    out = torch.empty(3, dtype=torch.float32, device=dev)
    c, p = make_config(cfg, T), make_params(params)
    _check(load().moe_balance_loss(ctypes.byref(c), _ptr(x), ctypes.byref(p), _ptr(idx),
                                   _ptr(gates), _ptr(thr), _ptr(perm), _ptr(offsets),
                                   w_importance, w_load, _ptr(imp), _ptr(load_), _ptr(out),
                                   ws.ptr, ws.nbytes, _stream()), "moe_balance_loss")
    return imp, load_, out


class ForwardOut:
    """Output tensors of one moe_forward call; with save=True also the tensors
    the backward pass reads (thresholds, routing, expert outputs)."""

    def __init__(self, cfg: MoEConfig, T: int, device, balance: bool, save: bool = False):
        self.y = torch.empty((T, cfg.d_model), dtype=_act_dtype(cfg), device=device)
        self.topk_idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=device)
        self.topk_gate = torch.empty((T, cfg.top_k), dtype=torch.float32, device=device)
        self.counts = torch.empty(cfg.n_experts, dtype=torch.int32, device=device)
        self.importance = (torch.empty(cfg.n_experts, dtype=torch.float32, device=device)
                           if balance else None)
        self.load = (torch.empty(cfg.n_experts, dtype=torch.float32, device=device)
                     if balance else None)
        self.balance = torch.empty(3, dtype=torch.float32, device=device) if balance else None
        A = T * cfg.top_k
        flat = not cfg.hierarchical
        self.thr = (torch.empty((T, 2), dtype=torch.float32, device=device)
                    if save and flat else None)
        self.offsets = (torch.empty(cfg.n_experts + 1, dtype=torch.int32, device=device)
                        if save else None)
        self.perm = torch.empty(A, dtype=torch.int32, device=device) if save else None
        self.inv = torch.empty(A, dtype=torch.int32, device=device) if save else None
        self.y_sorted = (torch.empty((A, cfg.d_model), dtype=_act_dtype(cfg), device=device)
                         if save else None)

    def struct(self) -> moe_outputs:
        return moe_outputs(y=_ptr(self.y), topk_idx=_ptr(self.topk_idx),
                           topk_gate=_ptr(self.topk_gate), counts=_ptr(self.counts),
                           importance=_ptr(self.importance), load=_ptr(self.load),
                           balance=_ptr(self.balance), thr=_ptr(self.thr),
                           offsets=_ptr(self.offsets), perm=_ptr(self.perm), inv=_ptr(self.inv),
                           y_sorted=_ptr(self.y_sorted))

    def saved(self) -> moe_saved:
        """The moe_saved view of these outputs (needs save=True)."""
        return moe_saved(topk_idx=_ptr(self.topk_idx), topk_gate=_ptr(self.topk_gate),
                         thr=_ptr(self.thr), offsets=_ptr(self.offsets), perm=_ptr(self.perm),
                         inv=_ptr(self.inv), y_sorted=_ptr(self.y_sorted),
                         importance=_ptr(self.importance), load=_ptr(self.load))


class Forward:
    """A prepared moe_forward call: argument structs are built once, so that
    repeated calls (benchmarks, graph capture) only cross into the library."""

    def __init__(self, cfg: MoEConfig, x, params, noise, w_importance=1.0, w_load=1.0,
                 balance=True, ws: Optional[Workspace] = None, out: Optional[ForwardOut] = None,
                 save: bool = False):
        T = x.shape[0]
        self.cfg = cfg
        self._keep = (x, params, noise)
        self.ws = ws or workspace(cfg, T, x.device)
        self.out = out or ForwardOut(cfg, T, x.device, balance, save)
        self._c = make_config(cfg, T)
        self._p = make_params(params)
        self._n = make_noise(noise)
        self._o = self.out.struct()
        self._x = _ptr(x)
        self._wi, self._wl = float(w_importance), float(w_load)
        self._fn = load().moe_forward

    def __call__(self) -> ForwardOut:
        _check(self._fn(ctypes.byref(self._c), self._x, ctypes.byref(self._p),
                        ctypes.byref(self._n), self._wi, self._wl, ctypes.byref(self._o),
                        self.ws.ptr, self.ws.nbytes, _stream()), "moe_forward")
        return self.out


def forward(cfg: MoEConfig, x, params, noise, w_importance=1.0, w_load=1.0, balance=True,
            ws: Optional[Workspace] = None, save: bool = False) -> ForwardOut:
    return Forward(cfg, x, params, noise, w_importance, w_load, balance, ws, save=save)()


def forward_static(cfg: MoEConfig, x, params, noise, w_importance=1.0, w_load=1.0,
                   balance=True, save: bool = False) -> ForwardOut:
    """moe_forward_static: the layer with the library's static scratch
    instead of a workspace (no allocation inside the call; the outputs are
    allocated here, by the caller)."""
    T = x.shape[0]
    out = ForwardOut(cfg, T, x.device, balance, save)
    c, p, n, o = make_config(cfg, T), make_params(params), make_noise(noise), out.struct()
    _check(load().moe_forward_static(ctypes.byref(c), _ptr(x), ctypes.byref(p), ctypes.byref(n),
                                     float(w_importance), float(w_load), ctypes.byref(o),
                                     _stream()), "moe_forward_static")
    return out


def mask_workspace_size(cfg: MoEConfig, rows_per_expert: int,
                        tokens: Optional[int] = None) -> int:
    c = make_config(cfg, tokens)
    return int(load().moe_mask_workspace_size(ctypes.byref(c), int(rows_per_expert)))


class MaskOut:
    """Output tensors of one moe_forward_mask call (see include/moe.h)."""

    def __init__(self, cfg: MoEConfig, T: int, m: int, device, balance: bool):
        E, R = cfg.n_experts, cfg.n_experts * m
        i32 = dict(dtype=torch.int32, device=device)
        self.y = torch.empty((T, cfg.d_model), dtype=_act_dtype(cfg), device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(R, **i32)
        self.tok_offsets = torch.empty(T + 1, **i32)
        self.slot_expert = torch.empty(R, **i32)
        self.slot_gate = torch.empty(R, dtype=torch.float32, device=device)
        self.slot_row = torch.empty(R, **i32)
        f32 = dict(dtype=torch.float32, device=device)
        self.importance = torch.empty(E, **f32) if balance else None
        self.load = torch.empty(E, **f32) if balance else None
        self.balance = torch.empty(3, **f32) if balance else None

    def struct(self) -> moe_mask_outputs:
        return moe_mask_outputs(**{n: _ptr(getattr(self, n)) for n, _ in moe_mask_outputs._fields_})


def forward_mask(cfg: MoEConfig, x, params, noise, rows_per_expert: int, thresholds=None,
                 w_importance=1.0, w_load=1.0, balance=True,
                 ws: Optional[Workspace] = None) -> MaskOut:
    """moe_forward_mask: the batch mask (thresholds None) or the threshold
    mask (thresholds [E] float32) in place of KeepTopK."""
    T = x.shape[0]
    m = int(rows_per_expert)
    ws = ws or Workspace(mask_workspace_size(cfg, m, T), x.device)
    out = MaskOut(cfg, T, m, x.device, balance)
    c, p, n, o = make_config(cfg, T), make_params(params), make_noise(noise), out.struct()
    _check(load().moe_forward_mask(ctypes.byref(c), _ptr(x), ctypes.byref(p), ctypes.byref(n), m,
                                   _ptr(thresholds), float(w_importance), float(w_load),
                                   ctypes.byref(o), ws.ptr, ws.nbytes, _stream()),
           "moe_forward_mask")
    return out


def backward_workspace_size(cfg: MoEConfig, tokens: Optional[int] = None) -> int:
    c = make_config(cfg, tokens)
    return int(load().moe_backward_workspace_size(ctypes.byref(c)))


class Grads:
    """Gradient tensors of one moe_backward call."""

    def __init__(self, cfg: MoEConfig, T: int, device, tables: bool = True):
        dt = _act_dtype(cfg)
        E, d, h = cfg.n_experts, cfg.d_model, cfg.d_hidden
        self.dx = torch.empty((T, d), dtype=dt, device=device)
        self.dw_gate = torch.empty((E, d), dtype=dt, device=device) if tables else None
        self.dw_noise = (torch.empty((E, d), dtype=dt, device=device)
                         if tables and cfg.noisy else None)
        hier = cfg.hierarchical
        self.dbias = (torch.empty(E, dtype=torch.float32, device=device)
                      if tables and not hier else None)
        self.dw1 = torch.empty((E, h, d), dtype=dt, device=device) if tables else None
        self.dw3 = (torch.empty((E, h, d), dtype=dt, device=device)
                    if tables and cfg.ffn == "swiglu" else None)
        self.dw2 = torch.empty((E, d, h), dtype=dt, device=device) if tables else None
        G = cfg.n_groups
        self.dw_gate_p = torch.empty((G, d), dtype=dt, device=device) if tables and hier else None
        self.dw_noise_p = (torch.empty((G, d), dtype=dt, device=device)
                           if tables and hier and cfg.noisy else None)

    def struct(self) -> moe_grads:
        return moe_grads(**{n: _ptr(getattr(self, n)) for n, _ in moe_grads._fields_})


class Backward:
    """A prepared moe_backward call for the tensors a saving forward produced."""

    def __init__(self, cfg: MoEConfig, x, params, noise, fwd: ForwardOut, dy,
                 w_importance=1.0, w_load=1.0, ws: Optional[Workspace] = None,
                 grads: Optional[Grads] = None):
        T = x.shape[0]
        self._keep = (x, params, noise, fwd, dy)
        self.ws = ws or Workspace(backward_workspace_size(cfg, T), x.device)
        self.grads = grads or Grads(cfg, T, x.device)
        self._c = make_config(cfg, T)
        self._p = make_params(params)
        self._n = make_noise(noise)
        self._s = fwd.saved()
        self._g = self.grads.struct()
        self._x, self._dy = _ptr(x), _ptr(dy)
        self._wi, self._wl = float(w_importance), float(w_load)
        self._fn = load().moe_backward

    def __call__(self) -> Grads:
        _check(self._fn(ctypes.byref(self._c), self._x, ctypes.byref(self._p),
                        ctypes.byref(self._n), ctypes.byref(self._s), self._dy, self._wi,
                        self._wl, ctypes.byref(self._g), self.ws.ptr, self.ws.nbytes, _stream()),
               "moe_backward")
        return self.grads


def backward(cfg: MoEConfig, x, params, noise, fwd: ForwardOut, dy, w_importance=1.0,
             w_load=1.0, ws: Optional[Workspace] = None) -> Grads:
    return Backward(cfg, x, params, noise, fwd, dy, w_importance, w_load, ws)()
