"""moe_forward captured into a HIP graph: the layer reads no device data back to the host, so one
capture replays the whole step. Each replay, with eager launches and synchronisations in between,
must reproduce the eager output bit for bit."""
import pytest
import torch

from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu

CASES = {
    "mixtral_decode_mini": I.mini("mixtral_prefill", T=64, d=512, F=448),
    "deepseek_mini": I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192),
    "qwen_mini": I.mini("qwen3_30b_a3b", T=2000, d=256, F=192),
    "mixtral_T5000": I.mini("mixtral_prefill", T=5000, d=256, F=128),
}


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay(name):
    cfg = CASES[name]
    L = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"))
    L.forward()
    torch.cuda.synchronize()
    ref_y, ref_idx, ref_w = L.y.clone(), L.topk_idx.clone(), L.topk_w.clone()
    ref_counts = L.counts.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward()
    for rep in range(3):
        # eager work between replays: clobber every output, then run an eager stage
        L.y.fill_(float("nan"))
        L.topk_idx.fill_(-7)
        L.topk_w.fill_(float("nan"))
        L.counts.fill_(-7)
        L.route()
        torch.cuda.synchronize()
        L.topk_idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(L.y), bits(ref_y)), (name, rep)
        assert torch.equal(L.topk_idx, ref_idx) and torch.equal(L.counts, ref_counts), (name, rep)
        assert torch.equal(bits(L.topk_w), bits(ref_w)), (name, rep)
    print(f"[graph] {name}: 3 replays equal the eager forward", flush=True)
