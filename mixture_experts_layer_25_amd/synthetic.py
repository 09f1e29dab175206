"""Seeded synthetic inputs for the MoE layer forward.

This module only draws and encodes test inputs. It holds none of the layer's
arithmetic: no routing, no gating, no matmul. Both the CPU oracle and the GPU
path read the bytes it produces.

Recipe (every tensor, every config):

* Each tensor has a fixed id: x=1, W_r=2, bias/offset=3, W_gate=4, W_up=5,
  W_down=6, Ws_gate=7, Ws_up=8, Ws_down=9.
* Every tensor is drawn from its own PCG64 stream
  ``numpy.random.default_rng([seed, tensor_id, part])`` with ``standard_normal``
  in float32, scaled by the stated standard deviation. ``part`` is the expert
  index for per-expert weights (so experts can be drawn in parallel) and 0 for
  the other tensors.
* bf16 tensors are the float32 draw rounded to nearest-even (NaN never occurs).
* MXFP4 tensors (OCP Microscaling v1.0: e2m1 elements, one e8m0 scale per 32
  consecutive elements along the reduction dimension K) are quantised from the
  float32 draw: for each 32-block, X = 2^(floor(log2(amax)) - 2), each element
  v/X is rounded to the nearest e2m1 value with ties to the even code and
  saturated at +-6; an all-zero block gets scale code 0. Codes are stored by
  32-element K-blocks, block-major: ``codes uint8[E][K/32][N][16]`` (the 16
  bytes of block b of column n, element 2i of the block in the low nibble of
  byte i), ``scales uint8[E][K/32][N]``.

The five named workloads and their shapes come from the layer description:
a tiny fp32 top-2 layer, the Mixtral shape (8 experts, top-2, F=14336), a
capacity-limited top-2 layer with skewed logits, a fine-grained 128-expert
top-8 layer, and a 384-expert top-6 MXFP4 layer with one shared expert.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# dtype and gating codes; they mirror the C header's enums.
F32, BF16, MXFP4, MXFP4_A8 = 0, 1, 2, 3
# MXFP4_A8: the same MXFP4 weights; the routed experts' products take their
# activation operands (x rows, H) as MXFP8 blocks.


def is_mx(wdt: int) -> bool:
    return wdt in (MXFP4, MXFP4_A8)
GATE_SOFTMAX, GATE_SIGMOID, GATE_SQRT_SOFTPLUS = 0, 1, 2

TID_X, TID_WR, TID_BIAS = 1, 2, 3
TID_WG, TID_WU, TID_WD = 4, 5, 6
TID_SG, TID_SU, TID_SD = 7, 8, 9


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    D: int
    E: int
    k: int
    F: int
    act: int = BF16
    wdt: int = BF16
    gating: int = GATE_SOFTMAX
    renorm: int = 1
    capacity: int = 0          # <= 0: no limit
    clamp: float = 0.0         # <= 0: no clamp
    shared_F: int = 0          # 0: no shared expert
    bias: str = "none"         # "none" | "normal" | "linear"
    bias_sigma: float = 0.0
    x_sigma: float = 1.0
    wr_sigma: float = 0.02
    w_sigma: float = 0.02

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def capacity_int_formula(T: int, k: int, E: int) -> int:
    """Capacity as C integer code writes it: (T*k/E) in int, times 1.2,
    truncated on assignment to an int."""
    return int((T * k // E) * 1.2)


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", T=64, D=128, E=8, k=2, F=256,
                        act=F32, wdt=F32),
    "mixtral": Config("mixtral", T=4096, D=4096, E=8, k=2, F=14336,
                      bias="normal", bias_sigma=0.5),
    "capacity": Config("capacity", T=4096, D=4096, E=8, k=2, F=4096,
                       renorm=0, capacity=capacity_int_formula(4096, 2, 8),
                       bias="linear"),
    "fine128": Config("fine128", T=8192, D=4096, E=128, k=8, F=1536,
                      bias="normal", bias_sigma=1.0),
    "fine384_mxfp4": Config("fine384_mxfp4", T=16384, D=4096, E=384, k=6,
                            F=1024, wdt=MXFP4, gating=GATE_SQRT_SOFTPLUS,
                            renorm=0, clamp=10.0, shared_F=1024,
                            bias="normal", bias_sigma=0.1),
}
# The 384-expert layer with MXFP8 activation operands in the routed experts
# (an opt-in mode of the same weights; not one of the five workloads above).
CONFIGS["fine384_mxfp4_a8"] = CONFIGS["fine384_mxfp4"].replace(name="fine384_mxfp4_a8",
                                                               wdt=MXFP4_A8)
CONFIG_ORDER = ["tiny_fp32", "mixtral", "capacity", "fine128", "fine384_mxfp4"]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal(seed: int, tid: int, part: int, n: int, sigma: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, part])
    a = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


_E2M1_UP = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def quantize_mxfp4_rows(w_nk: np.ndarray):
    """Quantise rows of a float32 [N, K] matrix to MXFP4 along K.

    Returns (codes uint8[N, K/2], scales uint8[N, K/32]).
    """
    N, K = w_nk.shape
    assert K % 32 == 0
    blk = w_nk.reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    # floor(log2(amax)) from the float32 exponent field (amax > 0 normal).
    ebits = ((amax.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32)
    e_unb = ebits - 127
    sexp = np.where(amax > 0, e_unb - 2, -127)
    scode = np.clip(sexp + 127, 0, 254).astype(np.uint8)
    inv = np.ldexp(np.float32(1.0), -(scode.astype(np.int32) - 127)).astype(np.float32)
    v = blk * inv[:, :, None]
    mag = np.abs(v)
    # ties go to the even code: at 0.25, 1.25, 2.5, 5.0 round down; at
    # 0.75, 1.75, 3.5 round up.
    code = np.zeros(mag.shape, dtype=np.uint8)
    code += (mag > 0.25)
    code += (mag >= 0.75)
    code += (mag > 1.25)
    code += (mag >= 1.75)
    code += (mag > 2.5)
    code += (mag >= 3.5)
    code += (mag > 5.0)
    sign = (v < 0) & (code > 0)
    code = code | (sign.astype(np.uint8) << np.uint8(3))
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scode)


@dataclasses.dataclass
class Inputs:
    """Host-side inputs. Floating tensors hold raw bits: float32 arrays for
    fp32, uint16 arrays for bf16. MXFP4 weights hold codes and scales."""
    cfg: Config
    x: np.ndarray            # [T, D]   f32 or u16(bf16 bits)
    W_r: np.ndarray          # [D, E]   f32
    bias: np.ndarray | None  # [E]      f32
    W_gate: np.ndarray | None = None   # [E, D, F] f32/u16
    W_up: np.ndarray | None = None     # [E, D, F]
    W_down: np.ndarray | None = None   # [E, F, D]
    S_gate: np.ndarray | None = None   # MXFP4: codes [E,D/32,F,16] in W_gate, scales [E,D/32,F]
    S_up: np.ndarray | None = None
    S_down: np.ndarray | None = None   # MXFP4: codes [E,F/32,D,16] in W_down, scales [E,F/32,D]
    Ws_gate: np.ndarray | None = None  # [D, Fs] u16
    Ws_up: np.ndarray | None = None
    Ws_down: np.ndarray | None = None  # [Fs, D] u16


def _act_encode(a: np.ndarray, dt: int) -> np.ndarray:
    if dt == F32:
        return a
    if dt == BF16:
        return f32_to_bf16_bits(a)
    raise ValueError(dt)


def make_bias(cfg: Config, seed: int = 0) -> np.ndarray | None:
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        return _normal(seed, TID_BIAS, 0, cfg.E, cfg.bias_sigma)
    if cfg.bias == "linear":
        # 2.0 for expert 0 falling linearly to 0 for the last expert
        e = np.arange(cfg.E, dtype=np.float32)
        return (np.float32(2.0) * (np.float32(cfg.E - 1) - e) / np.float32(cfg.E - 1)).astype(np.float32)
    raise ValueError(cfg.bias)


def make_expert_weights(cfg: Config, tid: int, K: int, N: int, seed: int = 0,
                        pool: ThreadPoolExecutor | None = None):
    """Per-expert [K, N] weights (logical layout). For MXFP4, returns
    (codes [E,K/32,N,16], scales [E,K/32,N]), stored by 32-element K-blocks,
    block-major; else one [E,K,N] array."""
    E = cfg.E

    def one(e):
        w = _normal(seed, tid, e, K * N, cfg.w_sigma).reshape(K, N)
        if is_mx(cfg.wdt):
            codes, scales = quantize_mxfp4_rows(np.ascontiguousarray(w.T))
            return (np.ascontiguousarray(codes.reshape(N, K // 32, 16).transpose(1, 0, 2)),
                    np.ascontiguousarray(scales.T))
        return _act_encode(w, cfg.wdt)

    own = pool is None
    if own:
        pool = ThreadPoolExecutor(_threads())
    try:
        parts = list(pool.map(one, range(E)))
    finally:
        if own:
            pool.shutdown()
    if is_mx(cfg.wdt):
        codes = np.stack([p[0] for p in parts])
        scales = np.stack([p[1] for p in parts])
        return codes, scales
    return np.stack(parts)


def make_linear_layer_inputs(T: int, D: int, E: int, n_out: int, seed: int = 0,
                             x_sigma: float = 1.0, wr_sigma: float = 0.02, w_sigma: float = 0.02):
    """Inputs of the dense-versus-MoE comparison with single-linear experts:
    x [T, D] bf16 bits, W_r [D, E] f32, expert weights [E, D, n_out] bf16
    bits and a dense weight [D, D] bf16 bits, all ~N(0, sigma)."""
    x = _act_encode(_normal(seed, TID_X, 0, T * D, x_sigma).reshape(T, D), BF16)
    W_r = _normal(seed, TID_WR, 0, D * E, wr_sigma).reshape(D, E)
    W_lin = np.stack([_act_encode(_normal(seed, TID_WD, e, D * n_out, w_sigma).reshape(D, n_out), BF16)
                      for e in range(E)])
    W_dense = _act_encode(_normal(seed, TID_WG, 0, D * D, w_sigma).reshape(D, D), BF16)
    return x, W_r, W_lin, W_dense


def make_inputs(cfg: Config, seed: int = 0, with_experts: bool = True) -> Inputs:
    x = _act_encode(_normal(seed, TID_X, 0, cfg.T * cfg.D, cfg.x_sigma).reshape(cfg.T, cfg.D), cfg.act)
    W_r = _normal(seed, TID_WR, 0, cfg.D * cfg.E, cfg.wr_sigma).reshape(cfg.D, cfg.E)
    inp = Inputs(cfg=cfg, x=x, W_r=W_r, bias=make_bias(cfg, seed))
    if not with_experts:
        return inp
    with ThreadPoolExecutor(_threads()) as pool:
        if is_mx(cfg.wdt):
            inp.W_gate, inp.S_gate = make_expert_weights(cfg, TID_WG, cfg.D, cfg.F, seed, pool)
            inp.W_up, inp.S_up = make_expert_weights(cfg, TID_WU, cfg.D, cfg.F, seed, pool)
            inp.W_down, inp.S_down = make_expert_weights(cfg, TID_WD, cfg.F, cfg.D, seed, pool)
        else:
            inp.W_gate = make_expert_weights(cfg, TID_WG, cfg.D, cfg.F, seed, pool)
            inp.W_up = make_expert_weights(cfg, TID_WU, cfg.D, cfg.F, seed, pool)
            inp.W_down = make_expert_weights(cfg, TID_WD, cfg.F, cfg.D, seed, pool)
    if cfg.shared_F > 0:
        Fs = cfg.shared_F
        inp.Ws_gate = f32_to_bf16_bits(_normal(seed, TID_SG, 0, cfg.D * Fs, cfg.w_sigma).reshape(cfg.D, Fs))
        inp.Ws_up = f32_to_bf16_bits(_normal(seed, TID_SU, 0, cfg.D * Fs, cfg.w_sigma).reshape(cfg.D, Fs))
        inp.Ws_down = f32_to_bf16_bits(_normal(seed, TID_SD, 0, Fs * cfg.D, cfg.w_sigma).reshape(Fs, cfg.D))
    return inp


def small_variant(cfg: Config, T: int, D: int | None = None, F: int | None = None,
                  E: int | None = None, k: int | None = None, **kw) -> Config:
    """The same modes at a size the oracle finishes in seconds."""
    E = cfg.E if E is None else E
    k = cfg.k if k is None else k
    rep = dict(name=cfg.name + "_small", T=T, D=cfg.D if D is None else D,
               F=cfg.F if F is None else F, E=E, k=k)
    if cfg.shared_F:
        rep["shared_F"] = kw.pop("shared_F", 64 if F is None else F)
    if cfg.capacity > 0 and "capacity" not in kw:
        rep["capacity"] = capacity_int_formula(T, k, E)
    rep.update(kw)
    return cfg.replace(**rep)
