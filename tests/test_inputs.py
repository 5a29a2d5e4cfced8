"""Seeded input generators: determinism, prefix independence, recipe properties (CPU)."""
import numpy as np
import torch

from sparse_routing_expert_amd import inputs as I


def test_deterministic_and_prefix_independent():
    cfg = I.mini("small_bf16", T=200, d=64, F=64)
    a = I.gen_x(cfg, seed=0)
    b = I.gen_x(cfg, seed=0)
    assert torch.equal(a, b)
    short = I.gen_x(cfg.with_sizes(T=70), seed=0)
    assert torch.equal(short, a[:70])
    part = I.gen_x(cfg, seed=0, rows=slice(65, 130))
    assert torch.equal(part, a[65:130])
    assert not torch.equal(I.gen_x(cfg, seed=1), a)


def test_decode_rows_are_prefill_prefix():
    dec = I.CONFIGS["mixtral_decode"]
    pre = I.CONFIGS["mixtral_prefill"]
    assert torch.equal(I.gen_x(dec), I.gen_x(pre, rows=slice(0, 64)))


def test_expert_streams_independent_of_E():
    cfg = I.mini("small_bf16", T=8, d=64, F=32)
    w1 = I.gen_expert(cfg, 3)[0]
    w2 = I.gen_expert(cfg.with_sizes(E=4, d=64, F=32), 3)[0]
    assert torch.equal(w1, w2)


def test_dtypes_and_shapes():
    for name in ("tiny_fp32",):
        cfg = I.CONFIGS[name]
        L = I.gen_layer(cfg)
        assert L["x"].dtype == torch.float32 and L["x"].shape == (64, 64)
        assert L["w_in"].shape == (4, 128, 64) and L["b_in"].shape == (4, 128)
        assert L["w_out"].shape == (4, 64, 128) and L["b_out"].shape == (4, 64)
        assert L["w_r"].dtype == torch.float32 and L["sel_bias"] is None
    cfg = I.mini("deepseek_v3", T=16, d=64, F=32, Fs=32, E=16)
    L = I.gen_layer(cfg)
    assert L["x"].dtype == torch.bfloat16 and L["w_in"].shape == (16, 64, 64)
    assert L["ws_in"].shape == (64, 64) and L["ws_out"].shape == (64, 32)


def test_selection_bias_on_grid():
    cfg = I.CONFIGS["deepseek_v3"]
    _, b = I.gen_router(cfg.with_sizes(d=8))
    steps = b.double() / I.BIAS_STEP
    assert torch.allclose(steps, steps.round(), atol=1e-4)
    assert steps.round().abs().max() <= I.BIAS_STEPS


def test_zipf_router_rows():
    cfg = I.CONFIGS["qwen3_30b_a3b"].with_sizes(d=32)
    w, _ = I.gen_router(cfg)
    norms = w.norm(dim=1)
    assert int((norms == 0).sum()) == I.ZIPF_EMPTY
    perm = I.zipf_rank_to_expert(cfg)
    ranked = norms[perm[: cfg.E - I.ZIPF_EMPTY]]
    # scales decrease with rank (ties only inside the capped head)
    sc = np.array(I.zipf_router_scales(cfg.E - I.ZIPF_EMPTY, cfg.k))
    assert np.all(np.diff(sc) <= 1e-9) and ranked[0] > ranked[-1]
    t = I.zipf_targets(cfg.E - I.ZIPF_EMPTY, cfg.k)
    assert abs(t.sum() - cfg.k) < 1e-9 and t.max() <= I.ZIPF_CAP + 1e-12
