"""Token matrices at the 2 GiB edge of the forward's gathered up projection.

moe_forward reads token rows straight from x through sorted_token while x is below 2 GiB (the
buffer descriptor that spans x keeps the offset 2^31 out of range for rows past a group's end), and
otherwise writes x_perm as the stage calls do. One layer sits just below the edge (x = 2^31 - 16384
bytes, the gathered form, with rows near the end of x), one exactly on it (the copied form). Each is
checked three ways: the forward equals the stage calls (route, permute with the row copy, grouped
FFN, combine) bit for bit, every assignment's position and x_perm row is checked, and 64
tokens (the first, the last and 62 seeded picks) match the oracle evaluated on the GPU's selection.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = {
    "x_below_2GiB_gathered": I.mini("mixtral_prefill", T=131071, d=8192, F=64),
    "x_2GiB_copied": I.mini("mixtral_prefill", T=131072, d=8192, F=64),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_large_token_matrix(name):
    cfg = CASES[name]
    x_bytes = cfg.T * cfg.d * 2
    print(f"[large] {name}: T={cfg.T} d={cfg.d} x = {x_bytes} bytes (2^31 = {1 << 31})", flush=True)
    torch.manual_seed(0)
    lay = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"))
    t = lay.t
    lay.forward()
    torch.cuda.synchronize()
    y_fwd = lay.y.clone()
    idx_fwd, gw_fwd = lay.topk_idx.clone(), lay.topk_w.clone()
    lay.y.fill_(float("nan"))
    lay.route()
    lay.permute()
    lay.ffn()
    lay.combine()
    torch.cuda.synchronize()
    assert torch.equal(lay.topk_idx, idx_fwd) and torch.equal(lay.topk_w, gw_fwd)
    assert torch.equal(lay.y.view(torch.uint8), y_fwd.view(torch.uint8)), "forward != stages"
    # positions bit-exact against the oracle's permutation of the selection; x_perm compared on the GPU
    off, st, inv = R.permute(lay.topk_idx.cpu().numpy().astype(np.int64), cfg.E)
    assert (lay.offsets.cpu().numpy() == off).all()
    assert (lay.sorted_token.cpu().numpy() == st).all() and (lay.inv_pos.cpu().numpy() == inv).all()
    st_dev = torch.as_tensor(st, device="cuda")
    assert torch.equal(lay.x_perm.view(torch.int16), t["x"][st_dev].view(torch.int16)), "x_perm"
    del st_dev
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 62, replace=False)]))
    sel = torch.as_tensor(toks, device="cuda")
    idx = lay.topk_idx[sel].cpu().numpy().astype(np.int64)
    gates = R.f64(lay.topk_w[sel])
    ref = R.tokens_forward(t["x"][sel], idx, gates, P.get_expert_fn(lay), cfg.act)
    err = P.check_layer(cfg, y_fwd[sel], ref)
    print(f"[large] {name}: ok, {len(toks)} tokens, max per-token rel-L2 {err:.2e}", flush=True)
