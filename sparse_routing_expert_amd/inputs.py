"""Seeded synthetic inputs for the MoE-FFN layer forward.

This module draws the tensors a layer call consumes -- token activations,
router weights, the selection bias and the expert weights -- with the shapes,
dtypes and value distributions of the layers the pages discuss (a tiny fp32
GELU layer, a small bf16 SwiGLU layer, and Mixtral-, Qwen3-MoE- and
DeepSeek-V3-shaped layers). It holds none of the layer's arithmetic: no
router scores, no expert selection, no expert math. Both the HIP library
(through the tests and the benchmark) and the CPU oracle are fed from it.

Every tensor is drawn from its own counter-derived seed
(base seed, layer id, tensor id, expert or row-chunk), so one expert or one
block of token rows can be regenerated on its own, and the first rows of a
long token batch do not depend on its length.

Device: tensors are drawn with torch's generator on the device asked for.
CPU and GPU generators give different (equally valid) draws; a test feeds
the same tensors to both sides, so that never matters.
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Dict, Optional

import numpy as np
import torch

# --------------------------------------------------------------------------------------
# Layer descriptions
# --------------------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape and numeric recipe of one MoE-FFN layer (no arithmetic here)."""

    name: str
    T: int  # tokens
    d: int  # d_model
    F: int  # expert d_ff
    E: int  # routed experts
    k: int  # experts per token
    dtype: str  # "f32" or "bf16": activations and expert weights (router is always fp32)
    act: str  # "gelu" (Linear+GELU+Linear with biases) or "swiglu" (no biases)
    score: str  # "softmax" or "sigmoid"
    renorm: bool  # gates renormalised over the selected k
    Fs: int = 0  # shared (always-on) SwiGLU expert d_ff; 0 = none
    router: str = "iid"  # "iid" | "zipf" | "biased"
    router_std: float = 0.02  # standard deviation of router weight entries
    x_from: Optional[str] = None  # take token rows from another layer's x (decode variant)
    layer_id: int = 0  # selects the seed stream

    @property
    def A(self) -> int:
        return self.T * self.k

    @property
    def n_in(self) -> int:
        """Rows of each expert's input projection: F (GELU) or 2F (gate then up, SwiGLU)."""
        return 2 * self.F if self.act == "swiglu" else self.F

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_sizes(self, **kw) -> "LayerConfig":
        """A reduced copy with the same recipe (used for parity cases the oracle finishes fast)."""
        kw.setdefault("name", self.name + "_mini")
        kw.setdefault("x_from", None)
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, LayerConfig] = {
    # Tiny fp32 layer: router Linear(64->4, no bias), softmax over the selected top-2 logits,
    # experts Linear(64->128)+GELU+Linear(128->64) with biases; everything N(0, 1/fan_in).
    "tiny_fp32": LayerConfig("tiny_fp32", T=64, d=64, F=128, E=4, k=2, dtype="f32", act="gelu",
                             score="softmax", renorm=True, router_std=1.0 / 8.0, layer_id=1),
    # Small bf16 SwiGLU layer, roughly uniform routing.
    "small_bf16": LayerConfig("small_bf16", T=4096, d=1024, F=2816, E=16, k=2, dtype="bf16",
                              act="swiglu", score="softmax", renorm=True, layer_id=2),
    # Mixtral-8x7B-shaped layer, prefill and decode.
    "mixtral_prefill": LayerConfig("mixtral_prefill", T=8192, d=4096, F=14336, E=8, k=2,
                                   dtype="bf16", act="swiglu", score="softmax", renorm=True,
                                   layer_id=3),
    "mixtral_decode": LayerConfig("mixtral_decode", T=64, d=4096, F=14336, E=8, k=2, dtype="bf16",
                                  act="swiglu", score="softmax", renorm=True,
                                  x_from="mixtral_prefill", layer_id=3),
    # Qwen3-30B-A3B-shaped layer: skewed (capped-Zipf) popularity, 8 experts never chosen.
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", T=16384, d=2048, F=768, E=128, k=8,
                                 dtype="bf16", act="swiglu", score="softmax", renorm=True,
                                 router="zipf", layer_id=4),
    # DeepSeek-V3-shaped layer: sigmoid scores + selection-only bias, one shared expert.
    "deepseek_v3": LayerConfig("deepseek_v3", T=4096, d=7168, F=2048, E=256, k=8, dtype="bf16",
                               act="swiglu", score="sigmoid", renorm=True, Fs=2048,
                               router="biased", layer_id=5),
}

# Tensor ids of the seed streams.
_X, _WR, _BIAS, _WIN, _BIN, _WOUT, _BOUT, _SIN, _SOUT, _PERM, _WNOISE, _NOISE, _DY = range(13)
X_CHUNK_ROWS = 64  # token rows drawn per seed (so prefixes of x are length-independent)

ZIPF_S = 1.2  # popularity exponent of the Qwen3-shaped layer
ZIPF_EMPTY = 8  # experts that never receive a token in the Qwen3-shaped layer
ZIPF_CAP = 0.45  # largest token fraction one expert may receive (see zipf_targets)
BIAS_STEP = 0.001  # selection-bias grid step (the bias update step the pages quote)
BIAS_STEPS = 50  # |bias| <= BIAS_STEPS * BIAS_STEP


def _mix64(*vals: int) -> int:
    """splitmix64-style mixing of integers into one 63-bit seed."""
    h = 0x9E3779B97F4A7C15
    for v in vals:
        h = (h ^ (v & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h = (h + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h = z ^ (z >> 31)
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, *ids: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix64(*ids))
    return g


def _normal(shape, std: float, device, dtype: torch.dtype, *ids: int) -> torch.Tensor:
    """N(0, std^2) in fp32, then cast (bf16: round to nearest even) to `dtype`."""
    t = torch.randn(shape, generator=_gen(device, *ids), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


# --------------------------------------------------------------------------------------
# Capped-Zipf popularity (Qwen3-shaped layer)
# --------------------------------------------------------------------------------------


def zipf_targets(n_active: int, k: int, s: float = ZIPF_S, cap: float = ZIPF_CAP) -> np.ndarray:
    """Token fraction wanted for popularity ranks 1..n_active: min(cap, lam * r^-s), summing to k.

    With zero-mean token activations an expert lands in a token's top-k (k <= E/2)
    for at most half the tokens, so the Zipf head is capped just below 1/2.
    """
    r = np.arange(1, n_active + 1, dtype=np.float64)
    lo, hi = 0.0, 1e3
    for _ in range(200):
        lam = 0.5 * (lo + hi)
        if np.minimum(cap, lam * r ** -s).sum() > k:
            hi = lam
        else:
            lo = lam
    return np.minimum(cap, 0.5 * (lo + hi) * r ** -s)


def _membership_prob(c: np.ndarray, k: int, umax: float = 14.0, nu: int = 2801,
                     grad: Optional[np.ndarray] = None) -> np.ndarray:
    """P(expert e is among the k largest of independent N(0, c_j^2) draws), by quadrature.

    Gaussian order statistics, used only to size router rows. On a common
    threshold grid u >= 0, a Poisson-binomial recursion gives, for all experts
    together, the probability that exactly m < k draws exceed u; removing
    expert e's own factor (stable for u >= 0, where its exceedance probability
    is <= 1/2) leaves G_e(u) = P(fewer than k *other* draws exceed u). Then
    P_e = integral of the density of c_e*Z times G_e over u >= 0, plus the
    tail beyond the grid, where G_e is 1. Negative draws are never in the
    top k for k <= E/2 up to a negligible probability.
    """
    from scipy.special import ndtr

    n = c.size
    u = np.linspace(0.0, umax, nu)
    w = np.full(nu, umax / (nu - 1))
    w[0] *= 0.5
    w[-1] *= 0.5
    p = ndtr(-u[None, :] / c[:, None])  # [n, nu]: P(c_j Z > u)
    dp = np.zeros((nu, k))
    dp[:, 0] = 1.0
    for j in range(n):
        shifted = np.concatenate([np.zeros((nu, 1)), dp[:, :-1]], axis=1)
        dp = dp * (1.0 - p[j])[:, None] + shifted * p[j][:, None]
    out = np.empty(n)
    for e in range(n):
        q = p[e]
        g = np.empty((nu, k))
        g[:, 0] = dp[:, 0] / (1.0 - q)
        for m in range(1, k):
            g[:, m] = (dp[:, m] - g[:, m - 1] * q) / (1.0 - q)
        ge = np.clip(g.sum(axis=1), 0.0, 1.0)
        dens = np.exp(-0.5 * (u / c[e]) ** 2) / (c[e] * math.sqrt(2.0 * math.pi))
        out[e] = (dens * ge * w).sum() + ndtr(-umax / c[e])
        if grad is not None:  # d P_e / d log c_e with the other experts held fixed
            tail = math.exp(-0.5 * (umax / c[e]) ** 2) / math.sqrt(2.0 * math.pi) * umax / c[e]
            grad[e] = (dens * ((u / c[e]) ** 2 - 1.0) * ge * w).sum() + tail
    return out


@functools.lru_cache(maxsize=None)
def zipf_router_scales(n_active: int, k: int, s: float = ZIPF_S, cap: float = ZIPF_CAP) -> tuple:
    """Per-rank router-row scales c_r whose top-k membership matches zipf_targets (fixed point)."""
    target = zipf_targets(n_active, k, s, cap)
    logc = np.zeros(n_active)
    grad = np.empty(n_active)
    for _ in range(100):
        prob = _membership_prob(np.exp(logc), k, grad=grad)
        err = np.log(target) - np.log(np.maximum(prob, 1e-300))
        if np.max(np.abs(err)) < 2e-3:
            break
        sens = np.maximum(grad / np.maximum(prob, 1e-300), 0.05)  # d log P / d log c
        logc += np.clip(0.7 * err / sens, -0.5, 0.5)  # damped diagonal Newton step
        logc -= np.median(logc)
    return tuple(np.exp(logc).tolist())


# --------------------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------------------


def gen_x(cfg: LayerConfig, device="cpu", seed: int = 0, rows: Optional[slice] = None) -> torch.Tensor:
    """Token activations x ~ N(0,1) [T, d] in the layer dtype, drawn in 64-row chunks."""
    src = CONFIGS[cfg.x_from] if cfg.x_from else cfg
    T = cfg.T
    r0, r1 = (0, T) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else T)
    out = torch.empty((r1 - r0, cfg.d), dtype=cfg.torch_dtype, device=device)
    c0, c1 = r0 // X_CHUNK_ROWS, (r1 + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS
    for c in range(c0, c1):
        blk = _normal((X_CHUNK_ROWS, cfg.d), 1.0, device, cfg.torch_dtype, seed, src.layer_id, _X, c)
        a, b = max(r0, c * X_CHUNK_ROWS), min(r1, (c + 1) * X_CHUNK_ROWS)
        out[a - r0:b - r0] = blk[a - c * X_CHUNK_ROWS:b - c * X_CHUNK_ROWS]
    return out


def zipf_rank_to_expert(cfg: LayerConfig, seed: int = 0) -> torch.Tensor:
    """Seeded permutation: popularity rank r (0-based) -> expert id."""
    return torch.randperm(cfg.E, generator=_gen("cpu", seed, cfg.layer_id, _PERM))


def gen_router(cfg: LayerConfig, device="cpu", seed: int = 0):
    """Router weights W_r [E, d] fp32 and the selection bias [E] fp32 (or None)."""
    w = torch.empty((cfg.E, cfg.d), dtype=torch.float32, device=device)
    for e in range(cfg.E):
        w[e] = _normal((cfg.d,), cfg.router_std, device, torch.float32, seed, cfg.layer_id, _WR, e)
    bias = None
    if cfg.router == "zipf":
        n_active = cfg.E - ZIPF_EMPTY
        scales = zipf_router_scales(n_active, cfg.k)
        perm = zipf_rank_to_expert(cfg, seed)
        for r in range(cfg.E):
            e = int(perm[r])
            if r < n_active:
                w[e] *= scales[r]
            else:
                w[e].zero_()  # logit identically 0: never among a token's top-k
    elif cfg.router == "biased":
        steps = torch.randint(-BIAS_STEPS, BIAS_STEPS + 1, (cfg.E,),
                              generator=_gen("cpu", seed, cfg.layer_id, _BIAS))
        bias = (steps.to(torch.float64) * BIAS_STEP).to(torch.float32).to(device)
    return w, bias


def gen_noisy_router(cfg: LayerConfig, device="cpu", seed: int = 0, T: Optional[int] = None):
    """Noisy top-k inputs: the noise-scale projection W_noise [E, d] fp32 (same std as the router)
    and standard normal draws [T, E] fp32 (64-token chunks, like x)."""
    w = torch.empty((cfg.E, cfg.d), dtype=torch.float32, device=device)
    for e in range(cfg.E):
        w[e] = _normal((cfg.d,), cfg.router_std, device, torch.float32, seed, cfg.layer_id, _WNOISE, e)
    T = cfg.T if T is None else T
    n = torch.empty((T, cfg.E), dtype=torch.float32, device=device)
    for c0 in range(0, T, 64):
        c1 = min(T, c0 + 64)
        n[c0:c1] = _normal((c1 - c0, cfg.E), 1.0, device, torch.float32, seed, cfg.layer_id, _NOISE, c0 // 64)
    return w, n


def gen_dy(cfg: LayerConfig, device="cpu", seed: int = 0, T: Optional[int] = None) -> torch.Tensor:
    """Output gradient dy ~ N(0,1) [T, d] in the layer dtype (64-token chunks, like x)."""
    T = cfg.T if T is None else T
    out = torch.empty((T, cfg.d), dtype=cfg.torch_dtype, device=device)
    for c0 in range(0, T, X_CHUNK_ROWS):
        c1 = min(T, c0 + X_CHUNK_ROWS)
        out[c0:c1] = _normal((c1 - c0, cfg.d), 1.0, device, cfg.torch_dtype, seed, cfg.layer_id, _DY,
                             c0 // X_CHUNK_ROWS)
    return out


def gen_expert(cfg: LayerConfig, e: int, device="cpu", seed: int = 0):
    """One expert's weights: (w_in [n_in, d], b_in [F] | None, w_out [d, F], b_out [d] | None)."""
    dt = cfg.torch_dtype
    w_in = _normal((cfg.n_in, cfg.d), 1.0 / math.sqrt(cfg.d), device, dt, seed, cfg.layer_id, _WIN, e)
    w_out = _normal((cfg.d, cfg.F), 1.0 / math.sqrt(cfg.F), device, dt, seed, cfg.layer_id, _WOUT, e)
    b_in = b_out = None
    if cfg.act == "gelu":
        b_in = _normal((cfg.F,), 1.0 / math.sqrt(cfg.d), device, dt, seed, cfg.layer_id, _BIN, e)
        b_out = _normal((cfg.d,), 1.0 / math.sqrt(cfg.F), device, dt, seed, cfg.layer_id, _BOUT, e)
    return w_in, b_in, w_out, b_out


def gen_shared(cfg: LayerConfig, device="cpu", seed: int = 0):
    """Shared SwiGLU expert: (ws_in [2Fs, d], ws_out [d, Fs]) or (None, None)."""
    if not cfg.Fs:
        return None, None
    dt = cfg.torch_dtype
    ws_in = _normal((2 * cfg.Fs, cfg.d), 1.0 / math.sqrt(cfg.d), device, dt, seed, cfg.layer_id, _SIN, 0)
    ws_out = _normal((cfg.d, cfg.Fs), 1.0 / math.sqrt(cfg.Fs), device, dt, seed, cfg.layer_id, _SOUT, 0)
    return ws_in, ws_out


def gen_layer(cfg: LayerConfig, device="cpu", seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """All tensors of one layer call, stacked: w_in [E, n_in, d], w_out [E, d, F], ..."""
    x = gen_x(cfg, device, seed)
    w_r, sel_bias = gen_router(cfg, device, seed)
    dt = cfg.torch_dtype
    w_in = torch.empty((cfg.E, cfg.n_in, cfg.d), dtype=dt, device=device)
    w_out = torch.empty((cfg.E, cfg.d, cfg.F), dtype=dt, device=device)
    b_in = torch.empty((cfg.E, cfg.F), dtype=dt, device=device) if cfg.act == "gelu" else None
    b_out = torch.empty((cfg.E, cfg.d), dtype=dt, device=device) if cfg.act == "gelu" else None
    for e in range(cfg.E):
        wi, bi, wo, bo = gen_expert(cfg, e, device, seed)
        w_in[e] = wi
        w_out[e] = wo
        if b_in is not None:
            b_in[e] = bi
            b_out[e] = bo
    ws_in, ws_out = gen_shared(cfg, device, seed)
    return dict(x=x, w_r=w_r, sel_bias=sel_bias, w_in=w_in, b_in=b_in, w_out=w_out, b_out=b_out,
                ws_in=ws_in, ws_out=ws_out)


def mini(name: str, **sizes) -> LayerConfig:
    """Reduced parity case of a named layer: same recipe, sizes the oracle finishes in seconds."""
    return CONFIGS[name].with_sizes(**sizes)
