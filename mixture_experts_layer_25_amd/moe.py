"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function takes torch CUDA tensors, passes their device pointers and
torch's current HIP stream to the C ABI, and raises MoEError on a non-zero
status. All computation happens in libmoe's HIP kernels; there is no
fallback: if the library is not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

F32, BF16, MXFP4, MXFP4_A8 = 0, 1, 2, 3
GATE_SOFTMAX, GATE_SIGMOID, GATE_SQRT_SOFTPLUS = 0, 1, 2
WS_DISPATCH, WS_EXPERT_FFN, WS_FORWARD, WS_ROUTE = 0, 1, 2, 3

_GATING = {"softmax": GATE_SOFTMAX, "sigmoid": GATE_SIGMOID, "sqrt_softplus": GATE_SQRT_SOFTPLUS}
_DT = {"f32": F32, "fp32": F32, "bf16": BF16, "mxfp4": MXFP4, "mxfp4_a8": MXFP4_A8}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        super().__init__(f"{what} (status {status}{', hipError ' + str(hip_error) if hip_error else ''})")


class Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("F", ctypes.c_int32), ("top_k", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("clamp", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("shared_F", ctypes.c_int32)]

    def __repr__(self):
        return "Cfg(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("W_gate", "W_up", "W_down", "S_gate", "S_up", "S_down",
                 "Ws_gate", "Ws_up", "Ws_down")]


_lib = None
SYMBOLS = ["moe_workspace_size", "moe_route", "moe_dispatch", "moe_expert_ffn",
           "moe_expert_gate_up", "moe_expert_down",
           "moe_shared_expert", "moe_combine", "moe_forward", "moe_quantize_mxfp8",
           "moe_status_string", "moe_last_hip_error", "moe_version", "moe_set_split_wait",
           "moe_dispatch_noalloc", "moe_expert_gate_up_gathered",
           "moe_route_screened"]


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_25_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(Cfg)
    W = ctypes.POINTER(_Weights)
    L.moe_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
    L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.moe_route_screened.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_ffn.argtypes = [P, vp, vp, W, vp, vp, vp, sz, vp]
    L.moe_expert_gate_up.argtypes = [P, vp, vp, W, vp, vp, sz, vp]
    L.moe_expert_gate_up_gathered.argtypes = [P, vp, vp, vp, W, vp, vp, sz, vp]
    L.moe_expert_down.argtypes = [P, vp, vp, W, vp, vp, sz, vp]
    L.moe_shared_expert.argtypes = [P, vp, W, vp, vp, vp]
    L.moe_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_forward.argtypes = [P, vp, vp, vp, W, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_quantize_mxfp8.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_last_hip_error.restype = ctypes.c_int
    L.moe_version.restype = ctypes.c_int
    L.moe_set_split_wait.restype = ctypes.c_int
    L.moe_set_split_wait.argtypes = [ctypes.c_int]
    for name in ("moe_workspace_size", "moe_route", "moe_route_screened", "moe_dispatch",
                 "moe_dispatch_noalloc",
                 "moe_expert_ffn",
                 "moe_expert_gate_up", "moe_expert_gate_up_gathered", "moe_expert_down",
                 "moe_shared_expert", "moe_combine",
                 "moe_forward", "moe_quantize_mxfp8"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = lib()
        hip = L.moe_last_hip_error() if status == -4 else 0
        raise MoEError(status, L.moe_status_string(status).decode(), hip)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_cfg(T, D, E, F, top_k, gating="softmax", renorm=True, capacity=0, clamp=0.0,
             act="bf16", w="bf16", shared_F=0) -> Cfg:
    g = _GATING[gating] if isinstance(gating, str) else int(gating)
    a = _DT[act] if isinstance(act, str) else int(act)
    wd = _DT[w] if isinstance(w, str) else int(w)
    return Cfg(T, D, E, F, top_k, g, int(bool(renorm)), capacity, clamp, a, wd, shared_F)


def act_torch_dtype(cfg: Cfg):
    return torch.bfloat16 if cfg.act_dtype == BF16 else torch.float32


@dataclass
class Weights:
    """Device weights; keeps the tensors alive while the struct is used."""
    W_gate: torch.Tensor
    W_up: torch.Tensor
    W_down: torch.Tensor
    S_gate: torch.Tensor | None = None
    S_up: torch.Tensor | None = None
    S_down: torch.Tensor | None = None
    Ws_gate: torch.Tensor | None = None
    Ws_up: torch.Tensor | None = None
    Ws_down: torch.Tensor | None = None

    def struct(self) -> _Weights:
        return _Weights(*[_p(getattr(self, n)) for n in
                          ("W_gate", "W_up", "W_down", "S_gate", "S_up", "S_down",
                           "Ws_gate", "Ws_up", "Ws_down")])


def workspace_size(cfg: Cfg, kind: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(cfg), kind, ctypes.byref(n)))
    return n.value


def workspace(cfg: Cfg, kind: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(cfg, kind), 16), dtype=torch.uint8, device=device)


def route(cfg: Cfg, x, W_r, bias=None, topk_idx=None, topk_w=None, logits=None,
          want_logits=False, stream=None):
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    if logits is None and want_logits:
        logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
    _check(lib().moe_route(ctypes.byref(cfg), _p(x), _p(W_r), _p(bias), _p(topk_idx),
                           _p(topk_w), _p(logits), _stream(stream)))
    return topk_idx, topk_w, logits


def route_screened(cfg: Cfg, x, W_r, bias=None, topk_idx=None, topk_w=None, ws=None,
                   stream=None):
    """moe_route_screened: the same indices and weights as route(), with the
    MFMA screen and exact chains for the candidate experts only."""
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, WS_ROUTE, dev)
    _check(lib().moe_route_screened(ctypes.byref(cfg), _p(x), _p(W_r), _p(bias), _p(topk_idx),
                                    _p(topk_w), _p(ws), ws.numel(), _stream(stream)))
    return topk_idx, topk_w


def dispatch(cfg: Cfg, topk_idx, x, ws=None, stream=None, copy_rows=True):
    """moe_dispatch. x_perm is allocated in the activation dtype, [T*k, D];
    with MXFP4_A8 weights its bytes hold MXFP8 rows (codes, then grouped
    scales; see include/moe.h). copy_rows=False passes no x_perm (the rows
    are then gathered through perm by the gate/up GEMM)."""
    dev = x.device
    tk = cfg.T * cfg.top_k
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    # at least one row, so that no pointer is null at T = 0
    slot_pos = torch.empty((max(cfg.T, 1), cfg.top_k), dtype=torch.int32, device=dev)
    perm = torch.full((max(tk, 1),), -1, dtype=torch.int32, device=dev)
    x_perm = (torch.empty((max(tk, 1), cfg.D), dtype=act_torch_dtype(cfg), device=dev)
              if copy_rows else None)
    if ws is None:
        ws = workspace(cfg, WS_DISPATCH, dev)
    _check(lib().moe_dispatch(ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts), _p(offsets),
                              _p(slot_pos), _p(perm), _p(x_perm), _p(ws), ws.numel(),
                              _stream(stream)))
    return dict(counts=counts, offsets=offsets, slot_pos=slot_pos[:cfg.T], perm=perm,
                x_perm=x_perm)


def dispatch_noalloc(cfg: Cfg, topk_idx, x, counts, offsets, slot_pos, perm, x_perm,
                     stream=None):
    """moe_dispatch_noalloc: moe_dispatch into caller-allocated outputs, with
    the library's fixed device scratch instead of a workspace."""
    _check(lib().moe_dispatch_noalloc(ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts),
                                      _p(offsets), _p(slot_pos), _p(perm), _p(x_perm),
                                      _stream(stream)))


def expert_ffn(cfg: Cfg, x_perm, offsets, weights: Weights, H=None, y_perm=None, ws=None,
               stream=None):
    """moe_expert_ffn. H is allocated in the activation dtype, [T*k, F]; with
    MXFP4_A8 weights its bytes hold MXFP8 rows like x_perm."""
    dev = x_perm.device
    rows = max(cfg.T * cfg.top_k, 1)
    if H is None:
        H = torch.empty((rows, cfg.F), dtype=act_torch_dtype(cfg), device=dev)
    if y_perm is None:
        y_perm = torch.empty((rows, cfg.D), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(cfg, WS_EXPERT_FFN, dev)
    w = weights.struct()
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(offsets), ctypes.byref(w),
                                _p(H), _p(y_perm), _p(ws), ws.numel(), _stream(stream)))
    return H, y_perm


def expert_gate_up(cfg: Cfg, x_perm, offsets, weights: Weights, H, ws, stream=None, wstruct=None):
    w = wstruct if wstruct is not None else weights.struct()
    _check(lib().moe_expert_gate_up(ctypes.byref(cfg), _p(x_perm), _p(offsets), ctypes.byref(w),
                                    _p(H), _p(ws), ws.numel(), _stream(stream)))
    return H


def expert_gate_up_gathered(cfg: Cfg, x, perm, offsets, weights: Weights, H, ws, stream=None,
                            wstruct=None):
    w = wstruct if wstruct is not None else weights.struct()
    _check(lib().moe_expert_gate_up_gathered(ctypes.byref(cfg), _p(x), _p(perm), _p(offsets),
                                             ctypes.byref(w), _p(H), _p(ws), ws.numel(),
                                             _stream(stream)))
    return H


def expert_down(cfg: Cfg, H, offsets, weights: Weights, y_perm, ws, stream=None, wstruct=None):
    w = wstruct if wstruct is not None else weights.struct()
    _check(lib().moe_expert_down(ctypes.byref(cfg), _p(H), _p(offsets), ctypes.byref(w),
                                 _p(y_perm), _p(ws), ws.numel(), _stream(stream)))
    return y_perm


def quantize_mxfp8(x, codes=None, scales=None, stream=None):
    """bf16 rows [rows, K] -> MXFP8 (e4m3 codes uint8 [rows, K], e8m0
    scales uint8 [rows, K/32])."""
    rows, K = x.shape
    if codes is None:
        codes = torch.empty((max(rows, 1), K), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((max(rows, 1), K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_mxfp8(_p(x), rows, K, _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def shared_expert(cfg: Cfg, x, weights: Weights, H_shared=None, y_shared=None, stream=None):
    dev = x.device
    if H_shared is None:
        H_shared = torch.empty((max(cfg.T, 1), cfg.shared_F), dtype=torch.bfloat16, device=dev)
    if y_shared is None:
        y_shared = torch.empty((max(cfg.T, 1), cfg.D), dtype=torch.float32, device=dev)
    w = weights.struct()
    _check(lib().moe_shared_expert(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(H_shared),
                                   _p(y_shared), _stream(stream)))
    return H_shared, y_shared


def combine(cfg: Cfg, y_perm, slot_pos, topk_w, y_shared=None, y=None, stream=None):
    if y is None:
        y = torch.empty((max(cfg.T, 1), cfg.D), dtype=act_torch_dtype(cfg), device=y_perm.device)
    _check(lib().moe_combine(ctypes.byref(cfg), _p(y_perm), _p(slot_pos), _p(topk_w),
                             _p(y_shared), _p(y), _stream(stream)))
    return y


def forward(cfg: Cfg, x, W_r, bias, weights: Weights, y=None, ws=None, topk_idx=None,
            topk_w=None, counts=None, offsets=None, stream=None, wstruct=None):
    """The whole layer in one call (route, dispatch, experts, shared, combine)."""
    if y is None:
        y = torch.empty((max(cfg.T, 1), cfg.D), dtype=act_torch_dtype(cfg), device=x.device)
    if ws is None:
        ws = workspace(cfg, WS_FORWARD, x.device)
    w = wstruct if wstruct is not None else weights.struct()
    _check(lib().moe_forward(ctypes.byref(cfg), _p(x), _p(W_r), _p(bias), ctypes.byref(w),
                             _p(y), _p(topk_idx), _p(topk_w), _p(counts), _p(offsets), _p(ws),
                             ws.numel(), _stream(stream)))
    return y


def set_split_wait(polls: int) -> int:
    """moe_set_split_wait: polls of a split GEMM tile's ready flags before it
    stores NaN (process-wide); returns the previous value."""
    r = lib().moe_set_split_wait(int(polls))
    if r < 0:
        _check(r)
    return r
