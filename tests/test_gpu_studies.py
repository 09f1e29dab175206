"""GPU checks of the two comparisons built from the stage entry points:

* the MoE layer of single-linear experts (route -> dispatch -> grouped GEMM
  with K = D, N = n_out -> combine) against the oracle's routing and a plain
  float64 matrix product per selected expert ("ops-transformer MoE operator
  on Ascend NPU", the dense-versus-MoE comparison);
* the dense layer (the grouped GEMM with one expert holding every row)
  against a float64 matrix product;
* the shared expert added exactly once at top-k 1, 2 and 4 ("DeepSeek-V4.1-
  Flash fine-grained MoE (5A)", the top-k measurement), against the oracle
  and against the layer without the shared expert.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_25_amd import moe, studies, synthetic as syn, upload
from gpu_helpers import assert_close, check_routing, gpu_forward, tol_for

pytestmark = pytest.mark.gpu


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _f64(bits):
    return syn.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("T,D,E,k,n_out", [(300, 256, 8, 2, 64), (517, 128, 8, 1, 96)])
def test_linear_expert_moe_against_reference(T, D, E, k, n_out):
    print(f"[studies] linear MoE T={T} D={D} E={E} k={k} n_out={n_out}", flush=True)
    x_h, W_r_h, W_lin_h, _ = syn.make_linear_layer_inputs(T, D, E, n_out, seed=3)
    cfg = moe.make_cfg(T=T, D=D, E=E, F=n_out, top_k=k, gating="softmax", renorm=True)
    lin = studies.LinearMoE(cfg, _bf16_dev(x_h), torch.from_numpy(W_r_h).cuda(), None,
                            _bf16_dev(W_lin_h))
    y = lin()
    torch.cuda.synchronize()
    # routing: the oracle's, bit-exact
    scfg = syn.Config("lin", T=T, D=D, E=E, k=k, F=n_out)
    _, idx_ref, w_ref = oracle.route(scfg, x_h, W_r_h, None)
    assert np.array_equal(lin.idx.cpu().numpy(), idx_ref)
    assert np.allclose(lin.tw.cpu().numpy(), w_ref, rtol=1e-5, atol=1e-6)
    # y[t] = sum_j w[t][j] x_t W_{e_tj}, float64 from the bf16 inputs
    xd = _f64(x_h)
    Wd = _f64(W_lin_h)
    ref = np.zeros((T, n_out))
    for j in range(k):
        for e in range(E):
            sel = idx_ref[:, j] == e
            if sel.any():
                ref[sel] += w_ref[sel, j:j + 1].astype(np.float64) * (xd[sel] @ Wd[e])
    got = upload.to_host_bits(y)[:T]
    assert_close(got, syn.f32_to_bf16_bits(ref.astype(np.float32)), 2e-2, "linear-expert MoE")


def test_dense_linear_against_matmul():
    T, K, N = 300, 256, 192
    print(f"[studies] dense T={T} K={K} N={N}", flush=True)
    x_h, _, _, W_h = syn.make_linear_layer_inputs(T, K, 8, 64, seed=5)
    W_h = W_h[:, :N].copy()
    dense = studies.DenseLinear(_bf16_dev(x_h), _bf16_dev(W_h))
    y = dense().cpu().numpy()[:T].astype(np.float64)
    ref = _f64(x_h) @ _f64(W_h)
    err = np.abs(y - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() < 1e-4, err.max()


@pytest.mark.parametrize("k", [1, 2, 4])
def test_shared_expert_added_once_at_topk(k):
    cfg = syn.small_variant(syn.CONFIGS["fine384_mxfp4"], T=200, D=256, F=128, k=k).replace(
        name=f"shared_k{k}")
    print(f"[studies] shared expert once, {cfg}", flush=True)
    inp = syn.make_inputs(cfg)
    ref = oracle.forward(inp)
    got = gpu_forward(inp, stagewise=True)
    check_routing(cfg, got, ref)
    assert_close(got["y"], ref["y"], tol_for(cfg), cfg.name)
    # the same layer without the shared expert, and the shared expert alone
    c, x, W_r, bias, w = upload.to_device(inp)
    c_ns = moe.make_cfg(T=cfg.T, D=cfg.D, E=cfg.E, F=cfg.F, top_k=k, gating=cfg.gating,
                        renorm=bool(cfg.renorm), capacity=cfg.capacity, clamp=cfg.clamp,
                        act=cfg.act, w=cfg.wdt, shared_F=0)
    y_ns = moe.forward(c_ns, x, W_r, bias, w)
    _, y_sh = moe.shared_expert(c, x, w)
    y_all = moe.forward(c, x, W_r, bias, w)
    torch.cuda.synchronize()
    diff = (y_all.float() - y_ns.float()).cpu().numpy().astype(np.float64)
    sh = y_sh.cpu().numpy()[:cfg.T].astype(np.float64)
    # two bf16 roundings of outputs of magnitude |y| separate the two sides
    lim = 2e-2 * np.maximum(1.0, np.abs(sh)) + 2.0 ** -7 * np.abs(y_all.float().cpu().numpy())
    assert np.all(np.abs(diff - sh) <= lim)
