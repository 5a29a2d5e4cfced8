"""Noisy top-k gating on the GPU against the oracle: H = x W_r^T + noise * softplus(x W_noise^T)
with caller-supplied noise, then the same route checks as the plain router (selection on H with the
ambiguity protocol, H within the logit tolerance, gates, counts, statistics), and the layer output
through permute, grouped FFN and combine against the oracle on the same selection."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P
from tests.test_gpu_parity import poison

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_fp32": I.CONFIGS["tiny_fp32"],
    "mixtral_mini": I.mini("mixtral_prefill", T=700, d=512, F=448),
    # bf16 routers with at most 16 experts take the fused noisy kernel: 16 experts with a ragged last
    # block, and a token count past the one where the plain router switches to two token tiles a block
    "small_mini": I.mini("small_bf16", T=1234, d=512, F=256),
    "mixtral_T9000": I.mini("mixtral_prefill", T=9000, d=256, F=128),
    "qwen_T8192": I.mini("qwen3_30b_a3b", T=8192, d=128, F=64),
    "qwen_mini": I.mini("qwen3_30b_a3b", T=2000, d=256, F=192),
    "deepseek_mini": I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192),
    # d = 200 (a multiple of 8, not of 32): both projections through the router GEMM with a masked last
    # K stage, then the noisy selection
    "ragged_E8_d200": I.mini("mixtral_prefill", T=700, d=200, F=136),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noisy_route_and_layer(name):
    cfg = CASES[name]
    torch.manual_seed(0)
    L = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"))
    poison(L)
    w_n, noise = I.gen_noisy_router(cfg, device="cuda")
    t = L.t
    print(f"[noisy] {name}: T={cfg.T} E={cfg.E} k={cfg.k} {cfg.dtype} {cfg.score}", flush=True)
    ref = R.route(t["x"], t["w_r"], cfg.k, cfg.score, cfg.renorm, t["sel_bias"], w_n.cpu(), noise.cpu())
    L.route_noisy(w_n, noise)
    torch.cuda.synchronize()
    n_amb = P.check_route(cfg, L, ref)
    L.permute()
    L.ffn()
    if cfg.Fs:
        L.shared()
    L.combine()
    torch.cuda.synchronize()
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    g = R.gates(ref.logits, idx, cfg.score, cfg.renorm)
    off, st, inv = R.permute(idx, cfg.E)
    x64 = P.np64(t["x"])
    y_perm = R.experts_on_rows(x64[st], off, P.get_expert_fn(L), cfg.act)
    ys = R.shared_ffn(x64, P.np64(t["ws_in"]), P.np64(t["ws_out"])) if cfg.Fs else None
    y_ref = R.combine(y_perm, inv, g, ys)
    err = P.check_layer(cfg, L.y, y_ref)
    plain = R.route(t["x"], t["w_r"], cfg.k, cfg.score, cfg.renorm, t["sel_bias"])
    moved = int((np.sort(plain.idx, 1) != np.sort(ref.idx, 1)).any(1).sum())
    print(f"[noisy] {name}: ok ambiguous={n_amb} layer_err={err:.2e} tokens whose set the noise changed={moved}",
          flush=True)
    assert moved > 0  # the noise is strong enough to matter
