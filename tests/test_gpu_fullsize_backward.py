"""moe_backward on full-size layers, in the configuration the benchmark times (the forward stages,
then the backward with balancing coefficient 0.01), against the oracle where it can evaluate
outputs one by one:
  * dx and the router-logit gradient of sampled tokens (oracle tokens_backward on those tokens,
    plus the balancing term's rows from the whole layer's counts);
  * rows / columns of the expert weight gradients for sampled hidden features of the busiest, the
    least busy and (Qwen3-shaped layer) an empty expert (oracle expert_backward_features over the
    expert's full row set), and of the shared expert;
and through properties that hold at any size: dW_router = dlogits^T x, all gradients finite."""
import numpy as np
import pytest
import torch

from oracle import moe_grad as G
from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ["mixtral_prefill", "qwen3_30b_a3b", "deepseek_v3"]
N_TOKENS = {"mixtral_prefill": 8, "qwen3_30b_a3b": 8, "deepseek_v3": 4}
AUX = 0.01


def say(name, msg):
    print(f"[fullsize-backward] {name}: {msg}", flush=True)


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_backward(name):
    cfg = I.CONFIGS[name]
    tol = P.tol_for(cfg)
    say(name, "generating")
    tens = I.gen_layer(cfg, device="cuda")
    L = MoeLayer(cfg, tens)
    L.route()
    L.permute()
    L.ffn()
    if cfg.Fs:
        L.shared()
    L.combine()
    dy = I.gen_dy(cfg, device="cuda")
    g = L.alloc_grads()
    for v in g.values():
        if v is not None:
            v.fill_(float("nan"))
    L.backward(dy, g, aux_coef=AUX)
    torch.cuda.synchronize()
    say(name, "backward done")
    for key, v in g.items():
        if v is not None:
            assert torch.isfinite(v.float()).all(), f"{key} not finite"
    t = L.t
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    ref = R.route(t["x"], t["w_r"], cfg.k, cfg.score, cfg.renorm, t["sel_bias"])
    lg = L.logits.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(lg - ref.logits)) <= P.LOGIT_ATOL
    aux_dl = G.aux_backward(ref.logits, idx, cfg.score, AUX)
    get = R.stacked_experts(t["w_in"], t["b_in"], t["w_out"], t["b_out"])
    # property at any size: the router weight gradient is dlogits^T x
    dl_gpu = P.np64(g["dlogits"])
    x64 = P.np64(t["x"])
    P.grad_err(g["dw_r"], dl_gpu.T @ x64, cfg.E, "dw_router vs dlogits^T x", 1e-4)
    say(name, "router property ok")
    # sampled tokens
    rng = np.random.default_rng(1)
    S = np.sort(rng.choice(cfg.T, size=N_TOKENS[name], replace=False))
    dx_ref, dl_ref = G.tokens_backward(t["x"][torch.from_numpy(S).cuda()], t["w_r"], idx[S], ref.logits[S], get,
                                       cfg.act, cfg.score, cfg.renorm, t["ws_in"], t["ws_out"],
                                       dy[torch.from_numpy(S).cuda()], dl_extra=aux_dl[S])
    e_dx = P.grad_err(g["dx"][torch.from_numpy(S).cuda()], dx_ref, len(S), "dx (sampled tokens)", tol)
    e_dl = P.grad_err(dl_gpu[S], dl_ref, len(S), "dlogits (sampled tokens)", tol)
    say(name, f"sampled tokens ok dx={e_dx:.2e} dl={e_dl:.2e}")
    # sampled hidden features of chosen experts, over each expert's full row set
    off, st, inv = R.permute(idx, cfg.E)
    A = cfg.T * cfg.k
    row_t = np.empty(A, np.int64)
    row_j = np.empty(A, np.int64)
    row_t[inv] = np.arange(A) // cfg.k
    row_j[inv] = np.arange(A) % cfg.k
    gates = R.gates(ref.logits, idx, cfg.score, cfg.renorm)
    counts = np.diff(off)
    nonempty = np.nonzero(counts > 0)[0]
    experts = {int(nonempty[np.argmax(counts[nonempty])]), int(nonempty[np.argmin(counts[nonempty])])}
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        experts.add(int(empty[0]))
    F = cfg.F
    feats = np.unique(np.array([0, int(rng.integers(1, F - 1)), F - 1]))
    dy64 = P.np64(dy)
    for e in sorted(experts):
        rows = np.arange(off[e], off[e + 1])
        tt, jj = row_t[rows], row_j[rows]
        wi, bi, wo, bo = get(e)
        dwi, dbi, dwo = G.expert_backward_features(x64[tt], wi, bi, wo, bo, cfg.act,
                                                   gates[tt, jj][:, None] * dy64[tt], feats)
        gi = g["dw_in"][e]
        got_in = gi[torch.from_numpy(feats).cuda()] if cfg.act == "gelu" else \
            torch.cat([gi[torch.from_numpy(feats).cuda()], gi[torch.from_numpy(F + feats).cuda()]])
        e_in = P.grad_err(got_in, dwi, dwi.shape[0], f"dw_in expert {e}", tol)
        e_out = P.grad_err(g["dw_out"][e][:, torch.from_numpy(feats).cuda()].T, dwo.T, len(feats),
                           f"dw_out expert {e}", tol)
        if dbi is not None:
            P.grad_err(g["db_in"][e][torch.from_numpy(feats).cuda()], dbi, 1, f"db_in expert {e}", tol)
        say(name, f"expert {e} rows={rows.size} dw_in={e_in:.2e} dw_out={e_out:.2e}")
    if cfg.Fs:
        fs = np.unique(np.array([0, cfg.Fs // 2, cfg.Fs - 1]))
        dwi, _, dwo = G.expert_backward_features(x64, P.np64(t["ws_in"]), None, P.np64(t["ws_out"]), None, "swiglu",
                                                 dy64, fs)
        gi = g["dws_in"]
        got_in = torch.cat([gi[torch.from_numpy(fs).cuda()], gi[torch.from_numpy(cfg.Fs + fs).cuda()]])
        e_in = P.grad_err(got_in, dwi, dwi.shape[0], "dws_in", tol)
        e_out = P.grad_err(g["dws_out"][:, torch.from_numpy(fs).cuda()].T, dwo.T, len(fs), "dws_out", tol)
        say(name, f"shared expert ok dws_in={e_in:.2e} dws_out={e_out:.2e}")
