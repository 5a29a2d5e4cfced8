"""moe_backward on full-size layers, in the configuration the benchmark times (the forward stages,
then the backward with balancing coefficient 0.01), against the oracle:
  * dx of every token, row by row (relative L2 per token at the forward's tolerance, relative to the
    larger of the token's dx and the root-sum-square of the terms dx adds up), with the router term
    dlogits W_r formed from the GPU's logit gradient, and
    the router-logit gradient of every token (oracle tokens_backward over chunks of tokens, plus the
    balancing term's rows from the whole layer's counts);
  * the whole input and output projection gradients of the busiest expert, row by row (one hidden
    feature's input weights, one output feature's weights), over the expert's full row set (oracle
    expert_backward_features over every feature);
  * sampled hidden features of the least busy and (Qwen3-shaped layer) an empty expert, and of the
    shared expert;
and through properties that hold at any size: dW_router = dlogits^T x, all gradients finite.
A token's dx sums k expert terms, the shared expert's and the router's; where they cancel, the error
of each bf16-rounded term stays at the terms' scale, hence that denominator. The logit gradient is
gate_backward(dg) with dg = dy . y_perm: it must equal, to 1e-4 per token, the oracle's gate backward
of dg formed from the GPU's own bf16 y_perm, and every row of that y_perm must match the oracle's
per-expert loop at the layer tolerance. Against the all-float64 oracle the logit gradient's error is
y_perm's bf16 rounding amplified where a token's gate gradients cancel (two near-equal dg under a
dominant gate pair): its block measure (median floor) is held at the median and reported at the
99th percentile and maximum."""
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
CHUNK = 1024  # tokens per oracle call
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
    # every token, in chunks
    rng = np.random.default_rng(1)
    dx_gpu = P.np64(g["dx"])
    dx_ref = np.empty_like(dx_gpu)
    dl_ref = np.empty_like(dl_gpu)
    ssq = np.empty(cfg.T)
    for c0 in range(0, cfg.T, CHUNK):
        c1 = min(cfg.T, c0 + CHUNK)
        dx_ref[c0:c1], dl_ref[c0:c1], ssq[c0:c1] = G.tokens_backward(
            t["x"][c0:c1], t["w_r"], idx[c0:c1], ref.logits[c0:c1], get, cfg.act, cfg.score, cfg.renorm, t["ws_in"],
            t["ws_out"], dy[c0:c1], dl_extra=aux_dl[c0:c1], return_term_ssq=True)
    # dx = (expert and shared terms) + dlogits w_r. The logit gradient is checked on its own below;
    # the router term here uses the GPU's, so dx's rows measure the expert backward path
    w_r64 = P.np64(t["w_r"])
    dx_ref_g = dx_ref - dl_ref @ w_r64 + dl_gpu @ w_r64
    err_dx = P.sum_rel_l2(dx_gpu, dx_ref_g, ssq)
    err_dx_o = P.sum_rel_l2(dx_gpu, dx_ref, ssq)
    worst = int(np.argmax(err_dx))
    say(name, f"dx rows: max {err_dx.max():.2e} (token {worst}); with the oracle's logit gradient "
              f"max {err_dx_o.max():.2e} (token {int(np.argmax(err_dx_o))}), 99.9th pct {np.quantile(err_dx_o, 0.999):.2e}")
    assert err_dx.max() <= tol, f"dx: token {worst} rel-L2 {err_dx.max():.3g}"
    # The logit gradient is gate_backward(dg) with dg[t, j] = dy[t] . y_perm[row of (t, j)]: the GPU's
    # must equal the oracle's gate backward applied to dg formed (in float64) from the GPU's own bf16
    # y_perm, whose rows the forward checks hold to the layer tolerance. Against the all-float64
    # oracle the difference is y_perm's bf16 rounding, amplified where a token's gate gradients
    # cancel (two near-equal dg of a dominant gate pair): reported, and held to the block measure.
    inv = L.inv_pos.cpu().numpy().astype(np.int64).reshape(cfg.T, cfg.k)
    yp64 = P.np64(L.y_perm)
    dy64_all = P.np64(dy)
    dg_own = np.empty((cfg.T, cfg.k))
    for c0 in range(0, cfg.T, CHUNK):
        c1 = min(cfg.T, c0 + CHUNK)
        dg_own[c0:c1] = np.einsum("tkd,td->tk", yp64[inv[c0:c1]], dy64_all[c0:c1])
    dl_own = G.gate_backward(ref.logits, idx, cfg.score, cfg.renorm, dg_own) + aux_dl
    # scale of a token's logit gradient before its centring cancels: ||gates|| max_j |dg_j| (+ the
    # balancing term); the GPU's float32 dot products are exact to ~1e-6 of it
    gts = R.gates(ref.logits, idx, cfg.score, cfg.renorm)
    scale = np.linalg.norm(gts, axis=1) * np.abs(dg_own).max(axis=1) + np.linalg.norm(aux_dl, axis=1)
    e_own = np.linalg.norm(dl_gpu - dl_own, axis=1) / np.maximum(np.maximum(np.linalg.norm(dl_own, axis=1), scale),
                                                                 1e-300)
    assert e_own.max() <= 1e-4, f"dlogits vs the gate backward of its own y_perm: token {int(np.argmax(e_own))} " \
                                f"rel err {e_own.max():.3g}"
    num = np.linalg.norm(dl_gpu - dl_ref, axis=1)
    den = np.linalg.norm(dl_ref, axis=1)
    med = float(np.median(den[den > 0]))
    blk = num / np.maximum(den, med)
    say(name, f"dlogits: vs own-y_perm gate backward max {e_own.max():.2e}; vs float64 oracle block measure "
              f"median {np.median(blk):.2e}, 99th pct {np.quantile(blk, 0.99):.2e}, max {blk.max():.2e} "
              f"(token {int(np.argmax(blk))})")
    assert np.median(blk) <= tol, f"dlogits vs float64 oracle: median block error {np.median(blk):.3g}"
    # and the y_perm those dg come from: every row against the oracle's per-expert loop
    off_g = L.offsets.cpu().numpy().astype(np.int64)
    yp_ref = R.experts_on_rows(P.np64(L.x_perm), off_g, get, cfg.act)
    e_yp = R.rel_l2_per_row(yp64, yp_ref)
    assert e_yp.max() <= tol, f"y_perm: row {int(np.argmax(e_yp))} rel-L2 {e_yp.max():.3g}"
    e_dl = float(np.median(blk))
    say(name, f"every token ok dx={err_dx.max():.2e} dl(own)={e_own.max():.2e} y_perm={e_yp.max():.2e}")
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
    # the busiest expert's whole weight gradients, row by row
    busiest = int(nonempty[np.argmax(counts[nonempty])])
    rows = np.arange(off[busiest], off[busiest + 1])
    tt, jj = row_t[rows], row_j[rows]
    wi, bi, wo, bo = get(busiest)
    dwi, dbi, dwo = G.expert_backward_features(x64[tt], wi, bi, wo, bo, cfg.act, gates[tt, jj][:, None] * dy64[tt],
                                               np.arange(F))
    e_in = R.rel_l2_per_row(P.np64(g["dw_in"][busiest]), dwi)
    e_out = R.rel_l2_per_row(P.np64(g["dw_out"][busiest]), dwo)
    assert e_in.max() <= tol, f"dw_in expert {busiest}: row {int(np.argmax(e_in))} rel-L2 {e_in.max():.3g}"
    assert e_out.max() <= tol, f"dw_out expert {busiest}: row {int(np.argmax(e_out))} rel-L2 {e_out.max():.3g}"
    if dbi is not None:
        e_b = R.rel_l2_per_row(P.np64(g["db_in"][busiest])[None, :], dbi[None, :])
        assert e_b.max() <= tol, f"db_in expert {busiest}: rel-L2 {e_b.max():.3g}"
    say(name, f"whole expert {busiest} rows={rows.size} dw_in={e_in.max():.2e} dw_out={e_out.max():.2e}")
    for e in sorted(experts - {busiest}):
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
