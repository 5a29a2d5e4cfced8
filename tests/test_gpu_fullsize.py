"""Full-size layers in the launch configuration the benchmark times (moe_forward), checked against
the oracle: routing of every token (bit-exact on unambiguous tokens), the permutation of every
assignment (bit-exact), the layer output of sampled tokens (one expert converted to float64 at a
time), and properties that hold at any size."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ["small_bf16", "mixtral_prefill", "mixtral_decode", "qwen3_30b_a3b", "deepseek_v3"]
N_SAMPLE = {"small_bf16": 48, "mixtral_prefill": 24, "mixtral_decode": 24, "qwen3_30b_a3b": 24, "deepseek_v3": 6}


@pytest.mark.parametrize("name", NAMES)
def test_fullsize(name):
    cfg = I.CONFIGS[name]
    print(f"[fullsize] {name}: generating", flush=True)
    tens = I.gen_layer(cfg, device="cuda")
    L = MoeLayer(cfg, tens)
    L.y.fill_(float("nan"))
    L.forward()
    torch.cuda.synchronize()
    print(f"[fullsize] {name}: forward done", flush=True)
    y = L.y.float()
    assert torch.isfinite(y).all()
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    gw = L.topk_w.cpu().numpy().astype(np.float64)
    assert L.counts.sum().item() == cfg.T * cfg.k
    if cfg.renorm:
        assert np.abs(gw.sum(axis=1) - 1).max() < 1e-5
    # routing of every token against the oracle (logits are not an output of moe_forward)
    t = L.t
    ref = R.route(t["x"], t["w_r"], cfg.k, cfg.score, cfg.renorm, t["sel_bias"])
    n_amb = P.check_route(cfg, L, ref, logits=False)
    # permutation of every assignment (stage call on the forward's own selection)
    L.permute()
    torch.cuda.synchronize()
    P.check_permute(cfg, L, None)
    # sampled tokens: y[t] from the oracle with the GPU's selection and the oracle's gates for it
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(cfg.T, size=min(N_SAMPLE[name], cfg.T), replace=False))
    g_ref = R.gates(ref.logits[toks], idx[toks], cfg.score, cfg.renorm)
    get = R.stacked_experts(t["w_in"], t["b_in"], t["w_out"], t["b_out"])
    y_ref = R.tokens_forward(t["x"][torch.from_numpy(toks).cuda()], idx[toks], g_ref, get, cfg.act, t["ws_in"],
                             t["ws_out"])
    err = P.check_layer(cfg, L.y[torch.from_numpy(toks).cuda()], y_ref)
    print(f"[fullsize] {name}: ok ambiguous={n_amb} sampled={len(toks)} layer_err={err:.2e}", flush=True)
