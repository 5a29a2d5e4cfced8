"""bench.py's CPU baseline leg (CPU): the stage-by-stage oracle run is the oracle's layer."""
import numpy as np

import bench
from oracle import moe_ref as R
from sparse_routing_expert_amd import inputs as I


def test_oracle_stages_equal_layer_forward():
    # fp32 GELU with biases, and a sigmoid-scored layer with a selection bias and a shared expert
    for cfg in (I.CONFIGS["tiny_fp32"], I.mini("deepseek_v3", T=48, d=64, F=32, Fs=32, E=16)):
        t = I.gen_layer(cfg)
        y, sec = bench.oracle_stages(cfg, t, t["x"])
        ref = R.layer_forward(t["x"], t["w_r"], R.stacked_experts(t["w_in"], t["b_in"], t["w_out"], t["b_out"]),
                              cfg.k, cfg.act, cfg.score, cfg.renorm, t["sel_bias"], t["ws_in"], t["ws_out"])
        assert np.array_equal(y, ref.y), cfg.name
        assert set(sec) == {"route", "permute", "expert_ffn", "shared", "combine"}
        assert all(v >= 0.0 for v in sec.values())


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stdout
