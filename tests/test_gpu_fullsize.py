"""Full-size layers in the launch configuration the benchmark times (moe_forward), checked against
the oracle on every token:
  * the routing stage with its logits output (the full-K router product), bit-exact selection on
    unambiguous tokens, gates, counts and statistics;
  * the forward's own routing, the same way;
  * the layer output of every token, against the oracle layer re-run on the forward's selection;
  * the permutation of every assignment (bit-exact) and every expert-output row y_perm of the
    stage calls (permute, grouped FFN), against the oracle's per-expert loop on the same rows;
  * the shared expert's output of every token where the layer has one.
The oracle converts one expert to float64 at a time, so the largest layer fits the host."""
import time

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ["small_bf16", "mixtral_prefill", "mixtral_decode", "qwen3_30b_a3b", "deepseek_v3"]


def _say(name, what, t0):
    print(f"[fullsize] {name}: {what} ({time.time() - t0:.1f} s)", flush=True)


@pytest.mark.parametrize("name", NAMES)
def test_fullsize(name):
    t0 = time.time()
    cfg = I.CONFIGS[name]
    _say(name, "generating", t0)
    tens = I.gen_layer(cfg, device="cuda")
    L = MoeLayer(cfg, tens)
    t = L.t
    sel_bias = None if t["sel_bias"] is None else R.f64(t["sel_bias"])
    ref = R.route(t["x"], t["w_r"], cfg.k, cfg.score, cfg.renorm, sel_bias)
    _say(name, "oracle route done", t0)

    # routing stage with logits: the full-K router product on every token
    L.logits.fill_(float("nan"))
    L.route(with_logits=True)
    torch.cuda.synchronize()
    n_amb = P.check_route(cfg, L, ref, logits=True)
    _say(name, f"route stage ok (ambiguous tokens: {n_amb})", t0)

    # the forward, as the benchmark runs it
    L.y.fill_(float("nan"))
    L.forward()
    torch.cuda.synchronize()
    assert torch.isfinite(L.y.float()).all()
    assert L.counts.sum().item() == cfg.T * cfg.k
    P.check_route(cfg, L, ref, logits=False)
    idx = L.topk_idx.cpu().numpy().astype(np.int64)
    _say(name, "forward routing ok", t0)

    # every token of the layer output against the oracle on the forward's selection
    lay = R.layer_forward(t["x"], t["w_r"], P.get_expert_fn(L), cfg.k, cfg.act, cfg.score, cfg.renorm, sel_bias,
                          t["ws_in"], t["ws_out"], forced_idx=idx)
    _say(name, "oracle layer done", t0)
    err_y = P.check_layer(cfg, L.y, lay.y)

    # stage calls on the same selection: permutation (bit-exact) and every y_perm row
    L.permute()
    torch.cuda.synchronize()
    off, _, _ = P.check_permute(cfg, L, None)
    assert (off == lay.offsets).all()
    L.y_perm.fill_(float("nan"))
    L.ffn()
    torch.cuda.synchronize()
    err_rows = R.rel_l2_per_row(P.np64(L.y_perm), lay.y_perm)
    assert err_rows.max() <= P.tol_for(cfg), f"y_perm max rel-L2 {err_rows.max():.3g}"
    err_sh = 0.0
    if cfg.Fs:
        L.y_shared.fill_(float("nan"))
        L.shared()
        torch.cuda.synchronize()
        err_sh = float(R.rel_l2_per_row(P.np64(L.y_shared), lay.y_shared).max())
        assert err_sh <= P.tol_for(cfg), f"shared expert max rel-L2 {err_sh:.3g}"
    _say(name, f"ok: ambiguous={n_amb} tokens={cfg.T} layer_err={err_y:.2e} y_perm_err={err_rows.max():.2e} "
               f"shared_err={err_sh:.2e}", t0)
