"""Writes outside any output or workspace buffer of the C ABI's calls.

Each output and each workspace sits inside a larger allocation whose margins (4 KB before and after)
hold a fixed byte pattern, and the workspaces are exactly the size `moe_workspace_bytes` asks for.
After the calls every margin must be unchanged. The parity tests poison outputs with NaN, which
catches elements left unwritten; this catches elements written out of bounds. The cases cover every
GEMM path (128- and 256-row eight-wave tiles, the wide-K kernel, the 64-row kernel, the fp32 kernel,
K-split tails, ragged widths), every route path (fused, logits kernel, router GEMM, noisy), expert
capacity, the shared expert, the bias step, the no-allocation permute and the backward.
"""
import pytest
import torch

from sparse_routing_expert_amd import _lib as L
from sparse_routing_expert_amd import inputs as I
from sparse_routing_expert_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5
TINY = I.CONFIGS["tiny_fp32"]

CASES = {
    "tiny_fp32": TINY.with_sizes(T=37),
    "T1": I.mini("deepseek_v3", T=1, d=128, F=64, Fs=64),
    "tiles128_small": I.mini("small_bf16", T=1000, d=256, F=320),
    "tiles256_ragged": I.mini("small_bf16", T=1300, d=264, F=328, E=4, k=2),
    "wide_ragged": I.mini("mixtral_prefill", T=8400, d=96, F=160),
    "decode_64row": I.mini("mixtral_prefill", T=64, d=200, F=456),
    "gelu_bias_ragged": TINY.with_sizes(dtype="bf16", T=300, d=72, F=200, E=6, k=2),
    "router_E40": I.mini("small_bf16", T=555, d=136, F=128, E=40, k=4),
    "deepseek_shared": I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192),
    "split_last_round": I.mini("small_bf16", T=1000, d=512, F=8448, E=1, k=1),
}
# the backward takes bf16 widths in multiples of 64
BWD_CASES = {
    "tiny_fp32": (TINY.with_sizes(T=37), 0.01),
    "small": (I.mini("small_bf16", T=1000, d=256, F=320), 0.0),
    "deepseek_shared": (I.mini("deepseek_v3", T=500, d=448, F=128, Fs=192), 0.001),
    "rows2100": (I.mini("small_bf16", T=2100, d=256, F=192, E=2, k=2), 0.01),
}


class Guarded:
    """A buffer of `nbytes` inside an allocation whose GUARD-byte margins hold PATTERN."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None):
        self.n = int(nbytes)
        self.raw = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        t = self.raw[GUARD:GUARD + self.n].view(dtype)
        self.t = t.view(shape) if shape is not None else t

    @classmethod
    def like(cls, x):
        return cls(x.numel() * x.element_size(), x.dtype, x.shape)

    def intact(self):
        return bool((self.raw[:GUARD] == PATTERN).all()) and bool((self.raw[GUARD + self.n:] == PATTERN).all())


OUTPUTS = ("logits", "topk_idx", "topk_w", "counts", "stats", "offsets", "sorted_token", "inv_pos", "x_perm",
           "y_perm", "y_shared", "y", "h")
STAGES = ("MOE_STAGE_ROUTE", "MOE_STAGE_ROUTE_NOISY", "MOE_STAGE_PERMUTE", "MOE_STAGE_FFN", "MOE_STAGE_EXPERT",
          "MOE_STAGE_SHARED", "MOE_STAGE_FORWARD", "MOE_STAGE_BACKWARD")


def guard_layer(lay):
    """Move the layer's outputs and workspaces into guarded allocations; returns the guards."""
    guards = {}
    for name in OUTPUTS:
        t = getattr(lay, name)
        if t is not None:
            g = Guarded.like(t)
            setattr(lay, name, g.t)
            guards[name] = g
    for stage_name in STAGES:
        stage = getattr(L, stage_name)
        n = L.moe_workspace_bytes(lay.shape, stage)
        g = Guarded(max(n, 1))
        lay._ws[stage] = g.t
        guards["ws:" + stage_name] = g
    return guards


def assert_intact(guards, what):
    torch.cuda.synchronize()
    bad = [k for k, g in guards.items() if not g.intact()]
    assert not bad, f"{what}: writes outside {bad}"


@pytest.mark.parametrize("name", sorted(CASES))
def test_no_writes_outside_buffers(name):
    cfg = CASES[name]
    print(f"[canary] {name}: T={cfg.T} d={cfg.d} F={cfg.F} E={cfg.E} k={cfg.k} {cfg.dtype} {cfg.act}", flush=True)
    torch.manual_seed(0)
    lay = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"))
    guards = guard_layer(lay)
    lay.route()
    lay.permute()
    lay.ffn()
    lay.up()
    lay.down()
    if cfg.Fs:
        lay.shared()
    lay.combine()
    assert_intact(guards, "stages")
    y_stages = lay.y.clone()
    lay.forward()
    assert_intact(guards, "forward")
    assert torch.equal(lay.y.view(torch.uint8), y_stages.view(torch.uint8)), "forward != stages"
    # noisy routing, the bias step and the no-allocation permute, on the same buffers
    w_n, noise = I.gen_noisy_router(cfg, device="cuda")
    lay.route_noisy(w_n, noise)
    assert_intact(guards, "noisy route")
    if lay.t["sel_bias"] is not None:
        bias = Guarded.like(lay.t["sel_bias"])
        bias.t.copy_(lay.t["sel_bias"])
        L.moe_update_bias(lay.shape, lay.counts, 1e-3, bias.t)
        assert_intact({"sel_bias": bias}, "bias step")
    L.moe_permute_noalloc(lay.shape, lay.topk_idx, lay.t["x"], lay.offsets, lay.sorted_token, lay.inv_pos,
                          lay.x_perm)
    assert_intact(guards, "no-allocation permute")


@pytest.mark.parametrize("name", ["tiles128_small", "deepseek_shared"])
def test_no_writes_outside_buffers_capacity(name):
    cfg = CASES[name]
    cap = max(1, cfg.T * cfg.k // cfg.E // 2)
    print(f"[canary] {name}: capacity {cap} rows per expert", flush=True)
    torch.manual_seed(0)
    lay = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"), capacity=cap)
    guards = guard_layer(lay)
    lay.route()
    lay.permute()
    lay.ffn()
    if cfg.Fs:
        lay.shared()
    lay.combine()
    lay.forward()
    assert_intact(guards, "capacity")


@pytest.mark.parametrize("name", sorted(BWD_CASES))
def test_no_writes_outside_buffers_backward(name):
    cfg, aux = BWD_CASES[name]
    print(f"[canary] backward {name}: T={cfg.T} d={cfg.d} F={cfg.F} E={cfg.E} k={cfg.k} {cfg.dtype}", flush=True)
    torch.manual_seed(0)
    lay = MoeLayer(cfg, I.gen_layer(cfg, device="cuda"))
    guards = guard_layer(lay)
    lay.route()
    lay.permute()
    lay.ffn()
    if cfg.Fs:
        lay.shared()
    lay.combine()
    grads = {}
    for k, v in lay.alloc_grads().items():
        if v is not None:
            g = Guarded.like(v)
            grads[k] = g.t
            guards["grad:" + k] = g
        else:
            grads[k] = None
    dy = I.gen_dy(cfg, device="cuda")
    lay.backward(dy, grads, aux_coef=aux)
    assert_intact(guards, "backward")
    for k, v in grads.items():
        if v is not None:
            assert bool(torch.isfinite(v).all()), k
