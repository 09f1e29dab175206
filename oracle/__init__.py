"""ctypes wrapper of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The GPU library neither imports nor links it.
Functions take numpy arrays (raw bits for bf16: uint16) and return numpy
arrays. Every function cites, in the C source, the page passage it follows.

Parity status per function (what pins it, see tests/test_oracle_*.py):
  router_logits   pinned: closed forms (zero rows, one-hot rows), float64 bound
  select_topk     pinned: brute-force rank count, tie rule, zero rows
  gate_weights    pinned: worked sqrt-softplus example, softplus tails,
                  softmax sums, renorm sums, the two top-k orderings;
                  sigmoid weights on non-zero logits with a selection bias
                  (renorm 0 and 1) against numpy's exp
  dispatch        pinned: invariants, capacity 1228, brute-force segments
  double_to_bf16  pinned: all 2^32 fp32 patterns against torch's conversion
  expert_rows     pinned: E=1,k=1 SwiGLU against a numpy matmul chain,
                  clamp closed form, dense-masked brute force
  shared_rows     pinned: numpy matmul chain over the decoded bf16 weights
                  with torch's bf16 rounding of H, shared_F != F, active clamp
  forward_tokens  pinned: dense all-experts masked brute force
  e4m3 / e4m3_encode / mxfp8_quantize
                  pinned: format values, exhaustive midpoints and ties,
                  torch's float8_e4m3fn rounding, block exponent, saturation,
                  round trips, error bound
  MXFP4_A8 experts pinned: numpy chain over the pinned quantiser
Full-size outputs are pinned only through the above (accumulation order,
exp/log1p ulps and bf16 ties of H are covered by the tolerance).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "moe_oracle.c")

OR_F32, OR_BF16, OR_MXFP4, OR_MXFP4_A8 = 0, 1, 2, 3
OR_SOFTMAX, OR_SIGMOID, OR_SQRT_SOFTPLUS = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, no fp contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("F", ctypes.c_int32), ("k", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("clamp", ctypes.c_float), ("act", ctypes.c_int32), ("wdt", ctypes.c_int32),
                ("shared_F", ctypes.c_int32)]


class _W(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("W_gate", "W_up", "W_down", "S_gate", "S_up", "S_down",
                 "Ws_gate", "Ws_up", "Ws_down")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        L = _lib
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_double_to_bf16_array.argtypes = [vp, ctypes.c_int64, vp]
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_uint]
        L.oracle_e8m0.restype = ctypes.c_double
        L.oracle_e8m0.argtypes = [ctypes.c_uint]
        L.oracle_e4m3.restype = ctypes.c_double
        L.oracle_e4m3.argtypes = [ctypes.c_uint]
        L.oracle_e4m3_encode.restype = ctypes.c_uint
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_mxfp8_quantize.argtypes = [vp, i32, vp, vp]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_capacity_formula.restype = i32
        L.oracle_capacity_formula.argtypes = [i32, i32, i32]
        P = ctypes.POINTER(_Cfg)
        W = ctypes.POINTER(_W)
        L.oracle_router_logits.argtypes = [P, vp, vp, vp]
        L.oracle_select_topk.argtypes = [P, vp, vp, vp]
        L.oracle_gate_weights.argtypes = [P, vp, vp, vp, vp]
        L.oracle_dispatch.argtypes = [P, vp, vp, vp, vp, vp]
        L.oracle_expert_rows.argtypes = [P, W, i32, i32, vp, vp, vp, vp]
        L.oracle_shared_rows.argtypes = [P, W, i32, vp, vp, vp]
        L.oracle_forward_tokens.argtypes = [P, W, vp, vp, vp, vp, i32, vp, vp, vp]
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def make_cfg(cfg) -> _Cfg:
    return _Cfg(cfg.T, cfg.D, cfg.E, cfg.F, cfg.k, cfg.gating, cfg.renorm, cfg.capacity,
                cfg.clamp, cfg.act, cfg.wdt, cfg.shared_F)


def _weights(inp) -> _W:
    return _W(*[_p(getattr(inp, n)) for n in
                ("W_gate", "W_up", "W_down", "S_gate", "S_up", "S_down",
                 "Ws_gate", "Ws_up", "Ws_down")])


# ---- scalar helpers -------------------------------------------------------
def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def double_to_bf16(v: float) -> int:
    return lib().oracle_double_to_bf16(float(v))


def double_to_bf16_array(v):
    """oracle_double_to_bf16 applied to every element of a float64 array."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_double_to_bf16_array(_p(v), v.size, _p(out))
    return out


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e8m0(s: int) -> float:
    return lib().oracle_e8m0(s)


def e4m3(code: int) -> float:
    return lib().oracle_e4m3(code)


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def mxfp8_quantize(v):
    """MXFP8 codes (uint8, same shape) and scales (uint8, last axis / 32) of
    float64 values whose last axis is a multiple of 32."""
    v = np.ascontiguousarray(v, np.float64)
    assert v.shape[-1] % 32 == 0
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    lib().oracle_mxfp8_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def mxfp8_values(codes, scales):
    """The values MXFP8 codes and scales represent (float64)."""
    dec = np.array([e4m3(c) for c in range(256)])
    sc = np.array([e8m0(s) if s < 255 else np.nan for s in range(256)])
    return dec[codes] * np.repeat(sc[scales], 32, axis=-1)


def softplus(s: float) -> float:
    return lib().oracle_softplus(s)


def silu(z: float) -> float:
    return lib().oracle_silu(z)


def capacity_formula(S: int, k: int, E: int) -> int:
    return lib().oracle_capacity_formula(S, k, E)


# ---- stages ---------------------------------------------------------------
def router_logits(cfg, x, W_r) -> np.ndarray:
    out = np.empty((cfg.T, cfg.E), np.float32)
    c = make_cfg(cfg)
    lib().oracle_router_logits(ctypes.byref(c), _p(x), _p(np.ascontiguousarray(W_r, np.float32)), _p(out))
    return out


def select_topk(cfg, logits, bias) -> np.ndarray:
    out = np.empty((cfg.T, cfg.k), np.int32)
    c = make_cfg(cfg)
    lib().oracle_select_topk(ctypes.byref(c), _p(logits), _p(bias), _p(out))
    return out


def gate_weights(cfg, logits, bias, idx) -> np.ndarray:
    out = np.empty((cfg.T, cfg.k), np.float32)
    c = make_cfg(cfg)
    lib().oracle_gate_weights(ctypes.byref(c), _p(logits), _p(bias), _p(idx), _p(out))
    return out


def route(cfg, x, W_r, bias):
    logits = router_logits(cfg, x, W_r)
    idx = select_topk(cfg, logits, bias)
    w = gate_weights(cfg, logits, bias, idx)
    return logits, idx, w


def dispatch(cfg, idx):
    c = make_cfg(cfg)
    counts = np.empty(cfg.E, np.int32)
    offsets = np.empty(cfg.E + 1, np.int32)
    slot_pos = np.empty((cfg.T, cfg.k), np.int32)
    perm = np.full(cfg.T * cfg.k, -1, np.int32)
    lib().oracle_dispatch(ctypes.byref(c), _p(np.ascontiguousarray(idx, np.int32)), _p(counts),
                          _p(offsets), _p(slot_pos), _p(perm))
    return counts, offsets, slot_pos, perm


def expert_rows(inp, expert: int, rows, want_h: bool = True, want_o: bool = True):
    cfg = inp.cfg
    rows = np.ascontiguousarray(rows, np.int32)
    n = len(rows)
    h = np.empty((n, cfg.F), np.float64) if want_h else None
    o = np.empty((n, cfg.D), np.float64) if want_o else None
    c = make_cfg(cfg)
    w = _weights(inp)
    lib().oracle_expert_rows(ctypes.byref(c), ctypes.byref(w), expert, n, _p(inp.x), _p(rows), _p(h), _p(o))
    return h, o


def shared_rows(inp, rows):
    cfg = inp.cfg
    rows = np.ascontiguousarray(rows, np.int32)
    o = np.empty((len(rows), cfg.D), np.float64)
    c = make_cfg(cfg)
    w = _weights(inp)
    lib().oracle_shared_rows(ctypes.byref(c), ctypes.byref(w), len(rows), _p(inp.x), _p(rows), _p(o))
    return o


def forward_tokens(inp, idx, w, slot_pos, tokens):
    """y rows for the listed tokens: (exact double [n, D], rounded act-dtype [n, D])."""
    cfg = inp.cfg
    tokens = np.ascontiguousarray(tokens, np.int32)
    n = len(tokens)
    y_exact = np.empty((n, cfg.D), np.float64)
    y_out = np.empty((n, cfg.D), np.float32 if cfg.act == OR_F32 else np.uint16)
    c = make_cfg(cfg)
    ww = _weights(inp)
    lib().oracle_forward_tokens(ctypes.byref(c), ctypes.byref(ww), _p(inp.x),
                                _p(np.ascontiguousarray(idx, np.int32)),
                                _p(np.ascontiguousarray(w, np.float32)),
                                _p(np.ascontiguousarray(slot_pos, np.int32)), n, _p(tokens),
                                _p(y_exact), _p(y_out))
    return y_exact, y_out


def forward(inp, tokens=None):
    """Whole layer: routing and dispatch on every token, y on ``tokens``
    (all tokens when None)."""
    cfg = inp.cfg
    logits, idx, w = route(cfg, inp.x, inp.W_r, inp.bias)
    counts, offsets, slot_pos, perm = dispatch(cfg, idx)
    if tokens is None:
        tokens = np.arange(cfg.T, dtype=np.int32)
    y_exact, y_out = forward_tokens(inp, idx, w, slot_pos, tokens)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                slot_pos=slot_pos, perm=perm, tokens=np.asarray(tokens, np.int32),
                y_exact=y_exact, y=y_out)
