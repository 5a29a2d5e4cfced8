"""moe_permute_noalloc (no workspace argument; scratch in a fixed array inside the library) against
moe_permute with a caller workspace, through the C ABI: every output bit-identical, and both equal
to the oracle's permutation. Each sequence makes two no-allocation calls in a row, the second with a
smaller input, so the second call runs on scratch the first one left behind."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_routing_expert_amd import _lib as L
from sparse_routing_expert_amd import inputs as I

pytestmark = pytest.mark.gpu

# (first, second) layers of each sequence; the permute paths: one-block index stage (A <= 2048),
# tiled ranks with offsets folded into the scatter (E <= 64, <= 64 tiles), tiled ranks with a
# separate scan (E > 64), and an expert capacity
SEQUENCES = {
    "scan_then_small": (I.mini("qwen3_30b_a3b", T=3000, d=128, F=64), I.mini("qwen3_30b_a3b", T=200, d=128, F=64)),
    "fold_then_fold": (I.mini("mixtral_prefill", T=9000, d=256, F=64), I.mini("mixtral_prefill", T=3100, d=256, F=64)),
    "scan_then_scan": (I.mini("deepseek_v3", T=4096, d=64, F=64, Fs=0), I.mini("deepseek_v3", T=1500, d=64, F=64,
                                                                                 Fs=0)),
}


def _routing(cfg, seed):
    """A valid selection (k distinct experts per token) drawn on the host, skewed toward low experts."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, cfg.E + 1) ** 0.7
    w /= w.sum()
    idx = np.stack([rng.choice(cfg.E, size=cfg.k, replace=False, p=w) for _ in range(cfg.T)]).astype(np.int32)
    return torch.from_numpy(idx).cuda()


def _buffers(cfg):
    A = cfg.T * cfg.k
    dev = "cuda"
    return dict(offsets=torch.full((cfg.E + 1,), -7, dtype=torch.int32, device=dev),
                sorted_token=torch.full((A,), -7, dtype=torch.int32, device=dev),
                inv_pos=torch.full((A,), -7, dtype=torch.int32, device=dev),
                x_perm=torch.full((A, cfg.d), float("nan"), dtype=cfg.torch_dtype, device=dev))


def _run_pair(cfg, capacity, seed):
    x = I.gen_x(cfg, device="cuda")
    idx = _routing(cfg, seed)
    shape = L.shape_of(cfg, capacity=capacity)
    ref = _buffers(cfg)
    ws = torch.empty((max(L.moe_workspace_bytes(shape, L.MOE_STAGE_PERMUTE), 1),), dtype=torch.uint8, device="cuda")
    L.moe_permute(shape, idx, x, ref["offsets"], ref["sorted_token"], ref["inv_pos"], ref["x_perm"], ws)
    got = _buffers(cfg)
    L.moe_permute_noalloc(shape, idx, x, got["offsets"], got["sorted_token"], got["inv_pos"], got["x_perm"])
    torch.cuda.synchronize()
    for name in ("offsets", "sorted_token", "inv_pos"):
        assert torch.equal(got[name], ref[name]), name
    assert torch.equal(got["x_perm"].view(torch.int16), ref["x_perm"].view(torch.int16)), "x_perm"
    # and both are the oracle's permutation of the same selection
    off, st, inv = R.permute(idx.cpu().numpy().astype(np.int64), cfg.E, capacity)
    n = int(off[-1])
    assert (got["offsets"].cpu().numpy() == off).all()
    assert (got["sorted_token"].cpu().numpy()[:n] == st).all()
    assert (got["inv_pos"].cpu().numpy() == inv).all()
    want = x.cpu()[torch.from_numpy(st)]
    assert torch.equal(got["x_perm"].cpu()[:n].view(torch.int16), want.view(torch.int16))
    return n


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_two_calls(name):
    first, second = SEQUENCES[name]
    assert second.T * second.k < first.T * first.k
    for i, cfg in enumerate((first, second)):
        print(f"[noalloc] {name} call {i}: T={cfg.T} E={cfg.E} k={cfg.k} d={cfg.d}", flush=True)
        n = _run_pair(cfg, 0, seed=10 * i + 1)
        print(f"[noalloc] {name} call {i}: ok rows={n}", flush=True)


def test_noalloc_capacity_two_calls():
    first = I.mini("qwen3_30b_a3b", T=2500, d=128, F=64)
    second = I.mini("qwen3_30b_a3b", T=900, d=128, F=64)
    for i, cfg in enumerate((first, second)):
        cap = R.capacity_rows(cfg.T, cfg.k, cfg.E, 1.0)
        print(f"[noalloc] capacity call {i}: T={cfg.T} C={cap}", flush=True)
        _run_pair(cfg, cap, seed=100 + i)
