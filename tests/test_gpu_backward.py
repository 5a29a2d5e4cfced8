"""moe_backward on the GPU against the float64 oracle's layer backward (oracle/moe_grad.py).

Each case runs the forward stages (route with logits, permute, grouped FFN, shared expert,
combine), then the backward through the C ABI, and compares every gradient -- dx, the router
weights, each expert's input and output projections (and biases), the shared expert and the router
logits -- with the oracle differentiating the same layer on the GPU's selection and expert capacity.
Cases: fp32 GELU with biases, bf16 GELU, SwiGLU with renormalised and raw softmax gates, skewed
routing with empty experts, sigmoid scoring with a selection bias and a shared expert, expert
capacity, the balancing-loss term, E = 1 with k = 1 and a single token. Sizes span several
128 x 128 tiles with ragged edges in every dimension.
"""
import numpy as np
import pytest
import torch

from oracle import moe_grad as G
from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P
from tests.test_gpu_parity import poison

pytestmark = pytest.mark.gpu

TINY = I.CONFIGS["tiny_fp32"]
# name: (layer, capacity factor or 0 for dropless, balancing coefficient)
CASES = {
    "tiny_fp32": (TINY, 0, 0.0),
    "tiny_fp32_aux": (TINY.with_sizes(T=37), 0, 0.01),
    "f32_swiglu_sigmoid_shared": (TINY.with_sizes(act="swiglu", score="sigmoid", router="biased", E=6, k=3, T=100,
                                                  Fs=64), 0, 0.01),
    "bf16_gelu_bias": (TINY.with_sizes(dtype="bf16", T=300, d=128, F=192, E=6, k=2), 0, 0.0),
    "small_mini": (I.mini("small_bf16", T=1000, d=256, F=320), 0, 0.0),
    "small_norenorm_aux": (I.mini("small_bf16", T=300, d=128, F=128, renorm=False), 0, 0.01),
    "mixtral_mini": (I.mini("mixtral_prefill", T=700, d=512, F=448), 0, 0.0),
    "mixtral_mini_c1.0": (I.mini("mixtral_prefill", T=700, d=512, F=448), 1.0, 0.0),
    "qwen_mini_aux": (I.mini("qwen3_30b_a3b", T=2000, d=256, F=192), 0, 0.01),
    "deepseek_mini": (I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192), 0, 0.0),
    "deepseek_mini_aux_c1.0": (I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192), 1.0, 0.001),
    "E1_k1": (I.mini("small_bf16", T=300, d=128, F=128, E=1, k=1), 0, 0.0),
    "T1": (I.mini("deepseek_v3", T=1, d=128, F=64, Fs=64), 0, 0.0),
    # at least 1536 rows per expert: the dgrad products run on the persistent GEMM against transposed
    # weights (SwiGLU, and GELU with biases, whose n_in = F)
    "rows1600_swiglu": (I.mini("small_bf16", T=1600, d=256, F=192, E=2, k=2), 0, 0.01),
    "rows1600_gelu_bias": (TINY.with_sizes(dtype="bf16", T=3200, d=128, F=192, E=2, k=1), 0, 0.0),
    # at least 2048 rows per expert: every grouped product, the fp32 dgrad ones included, runs on the
    # four-wave wide-K GEMM
    "rows2100_swiglu": (I.mini("small_bf16", T=2100, d=256, F=192, E=2, k=2), 0, 0.01),
}


def run_forward(L):
    L.route()
    L.permute()
    L.ffn()
    if L.cfg.Fs:
        L.shared()
    L.combine()
    torch.cuda.synchronize()


def poison_grads(g):
    for v in g.values():
        if v is not None:
            v.fill_(float("nan"))


def check_backward(name, cfg, L, dy, aux):
    tol = P.tol_for(cfg)
    print(f"[backward] {name}: T={L.T} d={cfg.d} F={cfg.F} E={cfg.E} k={cfg.k} {cfg.dtype} {cfg.act} {cfg.score} "
          f"C={L.capacity} aux={aux}", flush=True)
    g = L.alloc_grads()
    poison_grads(g)
    L.backward(dy, g, aux_coef=aux)
    torch.cuda.synchronize()
    t = L.t
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    ref = G.layer_backward(t["x"], P.np64(t["w_r"]), P.get_expert_fn(L), cfg.k, cfg.act, cfg.score, cfg.renorm,
                           None if t["sel_bias"] is None else P.np64(t["sel_bias"]), t["ws_in"], t["ws_out"], dy,
                           forced_idx=idx, capacity=L.capacity, aux_coef=aux)
    E, T = cfg.E, L.T
    errs = {
        "dx": P.grad_err(g["dx"], ref.dx, T, "dx", tol),
        "dlogits": P.grad_err(g["dlogits"], ref.dl, T, "dlogits", tol),
        "dw_r": P.grad_err(g["dw_r"], ref.dw_r, E, "dw_router", tol),
        "dw_in": P.grad_err(g["dw_in"], ref.dw_in, E, "dw_in", tol),
        "dw_out": P.grad_err(g["dw_out"], ref.dw_out, E, "dw_out", tol),
    }
    if ref.db_in is not None:
        errs["db_in"] = P.grad_err(g["db_in"], ref.db_in, E, "db_in", tol)
        errs["db_out"] = P.grad_err(g["db_out"], ref.db_out, E, "db_out", tol)
    if ref.dws_in is not None:
        errs["dws_in"] = P.grad_err(g["dws_in"], ref.dws_in, 2 * cfg.Fs, "dws_in", tol)
        errs["dws_out"] = P.grad_err(g["dws_out"], ref.dws_out, cfg.d, "dws_out", tol)
    # same inputs, same bits: every sum runs in a fixed order
    g2 = L.alloc_grads()
    poison_grads(g2)
    L.backward(dy, g2, aux_coef=aux)
    torch.cuda.synchronize()
    for key, v in g.items():
        if v is not None:
            assert torch.equal(v.view(torch.uint8), g2[key].view(torch.uint8)), f"{key} not deterministic"
    print(f"[backward] {name}: ok " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    return g, ref


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    cfg, factor, aux = CASES[name]
    torch.manual_seed(0)
    cap = R.capacity_rows(cfg.T, cfg.k, cfg.E, factor) if factor else 0
    L = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"), capacity=cap)
    poison(L)
    run_forward(L)
    dy = I.gen_dy(cfg, device="cuda")
    g, ref = check_backward(name, cfg, L, dy, aux)
    if cap:
        assert int((L.inv_pos.cpu().numpy() < 0).sum()) > 0, "capacity case drops nothing"
    if name.startswith("qwen"):
        empty = np.nonzero(L.counts.cpu().numpy() == 0)[0]
        assert empty.size > 0
        assert (g["dw_in"][empty] == 0).all() and (g["dw_out"][empty] == 0).all()
