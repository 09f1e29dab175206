"""Two comparisons the pages ask for, built from the library's stage entry
points (every step runs in the HIP kernels; this module only arranges the
calls and the buffers).

* Dense layer against an MoE layer of single-linear experts ("ops-transformer
  MoE operator on Ascend NPU", the performance comparison: S = 4096 tokens,
  D = 4096, 8 experts, top-2; the dense layer's 16.8 M weights are one
  4096 x 4096 matrix and the MoE's 4.2 M activated weights are two experts
  of 4096 x 512). Reading: an expert is one linear map x -> x W_e with
  W_e [D][n_out]; the layer output is y[t] = sum_j w[t][j] x_t W_{e_tj};
  the dense layer is y = x W, W [D][D]. Routing is the layer's softmax ->
  top-k -> renormalised router.
    - the linear experts are the grouped down-projection GEMM with K = D
      and N = n_out (moe_expert_down on the dispatched rows),
    - the dense layer is the same GEMM with one expert holding all T rows.

* Top-k sweep ("DeepSeek-V4.1-Flash fine-grained MoE (5A)", sec. 4,
  profiling: per-token time at top-k 1, 2, 4 for the same sequence length,
  with percentiles, and a record that checks the shared expert is not added
  twice); the sweep itself is bench.py --study topk. Reading: per-token
  time is step time / T over repeated steps (p50/p95/p99 over steps); the
  "top misses" are the (token, slot) pairs that the dispatch did not keep;
  the shared-expert check compares y(with shared) - y(without shared) with
  the shared expert's own output.
"""
from __future__ import annotations

import torch

from . import moe


def _cfg_like(c: moe.Cfg, **kw) -> moe.Cfg:
    d = {f: getattr(c, f) for f, _ in moe.Cfg._fields_}
    d.update(kw)
    return moe.Cfg(*[d[f] for f, _ in moe.Cfg._fields_])


def linear_weights(W: torch.Tensor) -> moe.Weights:
    """Weights struct whose down projection is W [E][K][N] (the gate/up
    slots, unused by the down stage, point at the same tensor)."""
    return moe.Weights(W_gate=W, W_up=W, W_down=W)


class LinearMoE:
    """MoE layer of single-linear experts: route -> dispatch -> grouped GEMM
    (K = D, N = n_out) -> combine, on device buffers allocated once."""

    def __init__(self, cfg: moe.Cfg, x, W_r, bias, W_lin: torch.Tensor):
        self.E, K, self.n_out = W_lin.shape
        assert K == cfg.D and self.E == cfg.E
        self.cfg = cfg
        # down stage: K (its "F") = D, N (its "D") = n_out
        self.cfg_lin = _cfg_like(cfg, F=cfg.D, D=self.n_out, shared_F=0)
        self.cfg_out = _cfg_like(cfg, D=self.n_out, F=cfg.D, shared_F=0)
        self.x, self.W_r, self.bias = x, W_r, bias
        self.w = linear_weights(W_lin)
        self.wstruct = self.w.struct()
        dev = x.device
        T, k = cfg.T, cfg.top_k
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.tw = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.d_ws = moe.workspace(cfg, moe.WS_DISPATCH, dev)
        self.f_ws = moe.workspace(self.cfg_lin, moe.WS_EXPERT_FFN, dev)
        self.y_perm = torch.empty((max(T * k, 1), self.n_out), dtype=torch.float32, device=dev)
        self.y = torch.empty((max(T, 1), self.n_out), dtype=moe.act_torch_dtype(cfg), device=dev)
        self.d = None

    def stages(self):
        """(name, callable) per stage, in order."""
        def route():
            moe.route(self.cfg, self.x, self.W_r, self.bias, self.idx, self.tw)

        def dispatch():
            self.d = moe.dispatch(self.cfg, self.idx, self.x, ws=self.d_ws)

        def experts():
            moe.expert_down(self.cfg_lin, self.d["x_perm"], self.d["offsets"], self.w,
                            self.y_perm, self.f_ws, wstruct=self.wstruct)

        def combine():
            moe.combine(self.cfg_out, self.y_perm, self.d["slot_pos"], self.tw, None, self.y)
        return [("route", route), ("dispatch", dispatch), ("experts", experts),
                ("combine", combine)]

    def __call__(self):
        for _, fn in self.stages():
            fn()
        return self.y


class DenseLinear:
    """y = x W (W [K][N]) as the grouped GEMM with one expert of all T rows."""

    def __init__(self, x: torch.Tensor, W: torch.Tensor, act="bf16"):
        T, K = x.shape
        K2, N = W.shape
        assert K == K2
        self.cfg = moe.make_cfg(T=T, D=N, E=1, F=K, top_k=1, act=act, w=act)
        self.x = x
        self.w = linear_weights(W.reshape(1, K, N))
        self.wstruct = self.w.struct()
        dev = x.device
        self.offsets = torch.tensor([0, T], dtype=torch.int32, device=dev)
        self.ws = moe.workspace(self.cfg, moe.WS_EXPERT_FFN, dev)
        self.y = torch.empty((max(T, 1), N), dtype=torch.float32, device=dev)

    def __call__(self):
        moe.expert_down(self.cfg, self.x, self.offsets, self.w, self.y, self.ws,
                        wstruct=self.wstruct)
        return self.y
